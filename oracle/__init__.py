"""CPU oracle for INT2/INT4 affine-quantised decode attention (fp64).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg load this; the GPU library never does. It shares no code with
the GPU library. The arithmetic lives in ``oracle.c`` (plain C, fp64); this
file only builds it with gcc and marshals numpy arrays through ctypes.

Format fields mirror the library's format (bits, K/V grouping axis, group
size, head_dim, KV/query heads, page size) because both describe the same
cache; the layout itself is implemented independently in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A test may point the loader at another build of oracle.c (a copy with a
# planted mistake, to show that the pins catch it); that build is used as is.
_LIB_OVERRIDE = os.environ.get("KVQ_ORACLE_LIB")

TOKEN_WISE, CHANNEL_WISE = 0, 1
_AXIS = {"token": TOKEN_WISE, "channel": CHANNEL_WISE, 0: TOKEN_WISE, 1: CHANNEL_WISE}


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
                               "-fPIC", "-shared", "-pthread", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Fmt(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("bits", "k_axis", "v_axis", "group", "head_dim",
                                               "num_kv_heads", "num_q_heads", "page_size")]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            L = ctypes.CDLL(_LIB)
        L.orc_f32_to_f16.restype = ctypes.c_uint16
        L.orc_f32_to_f16.argtypes = [ctypes.c_float]
        L.orc_f16_to_f64.restype = ctypes.c_double
        L.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_f64.restype = ctypes.c_double
        L.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _threads(n):
    return int(n) if n else min(16, os.cpu_count() or 1)


def make_format(bits, k_axis="channel", v_axis="token", group=128, head_dim=128, num_kv_heads=1,
                num_q_heads=4, page_size=0) -> _Fmt:
    return _Fmt(bits, _AXIS[k_axis], _AXIS[v_axis], group, head_dim, num_kv_heads, num_q_heads,
                page_size)


def fmt_of(w, group=128) -> _Fmt:
    """Format of a synth.Workload."""
    return make_format(w.bits, w.k_axis, w.v_axis, group, w.head_dim, w.num_kv_heads,
                       w.num_q_heads, w.page_size)


# ---- scalar conversions -------------------------------------------------

def f32_to_f16_bits(x) -> np.ndarray:
    x = np.asarray(x, np.float32)
    f = lib().orc_f32_to_f16
    return np.array([f(float(v)) for v in x.ravel()], np.uint16).reshape(x.shape)


def f16_bits_to_f64(h) -> np.ndarray:
    h = np.asarray(h, np.uint16)
    f = lib().orc_f16_to_f64
    return np.array([f(int(v)) for v in h.ravel()], np.float64).reshape(h.shape)


# ---- cache geometry -------------------------------------------------------

def padded_len(max_len: int) -> int:
    return ((max_len + 127) // 128) * 128


def cache_shapes(fmt: _Fmt, batch: int, max_len: int, num_pages: int = 0):
    """numpy (dtype, shape) of k_codes, v_words, k_sz, v_sz in the documented layout."""
    D, b, G, H = fmt.head_dim, fmt.bits, fmt.group, fmt.num_kv_heads
    tpw = 32 // b
    if fmt.page_size == 0:
        Lp = padded_len(max_len)
        kc = (np.uint8, (batch, H, Lp // 64, 64 * D * b // 8))
        vw = (np.uint32, (batch, H, Lp // 64, 64 // tpw * D))
        def sz(axis):
            return (np.uint16, (batch, H, Lp, D // G, 2) if axis == TOKEN_WISE
                    else (batch, H, Lp // G, D, 2))
    else:
        P = num_pages
        kc = (np.uint8, (P, H, 64 * D * b // 8))
        vw = (np.uint32, (P, H, 64 // tpw * D))
        def sz(axis):
            return (np.uint16, (P, H, 64, D // G, 2) if axis == TOKEN_WISE else (P, H, D, 2))
    return kc, vw, sz(fmt.k_axis), sz(fmt.v_axis)


def alloc_cache(fmt, batch, max_len, num_pages=0):
    return [np.zeros(shape, dt) for dt, shape in cache_shapes(fmt, batch, max_len, num_pages)]


# ---- the oracle's operations ----------------------------------------------

def quantize_group(x, bits):
    """(s_bits, z_bits, codes) for one group of float32 values."""
    x = np.ascontiguousarray(x, np.float32)
    codes = np.zeros(x.size, np.uint8)
    s = ctypes.c_uint16()
    z = ctypes.c_uint16()
    lib().orc_quantize_group(_p(x), ctypes.c_long(1), ctypes.c_int(x.size), ctypes.c_int(bits),
                             ctypes.byref(s), ctypes.byref(z), _p(codes), ctypes.c_long(1))
    return s.value, z.value, codes


def quantize_pack(fmt, k, v, seq_lens, page_table=None, num_pages=0, cache=None, threads=None):
    """Quantise + pack K, V ([B][Hkv][max_len][D] float32). Returns [k_codes, v_words, k_sz, v_sz]."""
    k = np.ascontiguousarray(k, np.float32)
    v = np.ascontiguousarray(v, np.float32)
    B, _, max_len, _ = k.shape
    lens = np.ascontiguousarray(seq_lens, np.int32)
    pt = None if page_table is None else np.ascontiguousarray(page_table, np.int32)
    maxp = 0 if pt is None else pt.shape[1]
    if cache is None:
        cache = alloc_cache(fmt, B, max_len, num_pages)
    rc = lib().orc_quantize_pack(ctypes.byref(fmt), _p(k), _p(v), _p(lens), _p(pt),
                                 ctypes.c_int(maxp), ctypes.c_int(B), ctypes.c_int(max_len),
                                 *[_p(c) for c in cache], ctypes.c_int(_threads(threads)))
    if rc != 0:
        raise ValueError("oracle: unsupported format")
    return cache


def dequantize_unit(fmt, which, cache, b, h, length, max_len, page_table=None):
    """[L][D] fp64 dequantised K ('k') or V ('v') of one (b, h)."""
    codes = cache[0] if which == "k" else cache[1]
    sz = cache[2] if which == "k" else cache[3]
    pt = None if page_table is None else np.ascontiguousarray(page_table, np.int32)
    out = np.zeros((max(length, 0), fmt.head_dim), np.float64)
    rc = lib().orc_dequantize_unit(ctypes.byref(fmt), ctypes.c_int(1 if which == "k" else 0),
                                   _p(codes), _p(sz), _p(pt),
                                   ctypes.c_int(0 if pt is None else pt.shape[1]),
                                   ctypes.c_int(max_len), ctypes.c_int(b), ctypes.c_int(h),
                                   ctypes.c_int(length), _p(out))
    if rc != 0:
        raise ValueError("oracle: unsupported format")
    return out


def attention_f64(q, kh, vh, scale):
    """softmax(scale * q.K^T).V in fp64; q [R][D], kh/vh [L][D]."""
    q = np.ascontiguousarray(q, np.float64)
    kh = np.ascontiguousarray(kh, np.float64)
    vh = np.ascontiguousarray(vh, np.float64)
    R, D = q.shape
    L = kh.shape[0]
    out = np.zeros((R, D), np.float64)
    lib().orc_attention_f64(_p(q), _p(kh), _p(vh), ctypes.c_int(L), ctypes.c_int(D),
                            ctypes.c_int(R), ctypes.c_double(scale), _p(out))
    return out


def decode_attention(fmt, q_bf16, cache, seq_lens, max_len, scale, page_table=None, units=None,
                     threads=None, out=None):
    """[B][Hq][D] fp64 decode attention over a packed cache (plain definition).

    units: optional list of (b, h) pairs; only those query heads are computed."""
    q = np.ascontiguousarray(q_bf16, np.uint16)
    B = q.shape[0]
    lens = np.ascontiguousarray(seq_lens, np.int32)
    pt = None if page_table is None else np.ascontiguousarray(page_table, np.int32)
    u = None if units is None else np.ascontiguousarray(np.asarray(units, np.int32).reshape(-1, 2))
    if out is None:
        out = np.zeros((B, fmt.num_q_heads, fmt.head_dim), np.float64)
    rc = lib().orc_decode_attention(ctypes.byref(fmt), _p(q), *[_p(c) for c in cache], _p(lens),
                                    _p(pt), ctypes.c_int(0 if pt is None else pt.shape[1]),
                                    ctypes.c_int(B), ctypes.c_int(max_len), ctypes.c_double(scale),
                                    _p(u), ctypes.c_int(0 if u is None else u.shape[0]), _p(out),
                                    ctypes.c_int(_threads(threads)))
    if rc != 0:
        raise ValueError("oracle: unsupported format")
    return out


def decode_attention_folded(fmt, q_bf16, cache, seq_lens, max_len, scale, page_table=None,
                            bug=False, threads=None):
    """The same output through the four folds, fp64 (cross-check of the algebra).

    bug=True accumulates acc-fold partials across group boundaries (a planted
    mistake the tests must detect)."""
    q = np.ascontiguousarray(q_bf16, np.uint16)
    B = q.shape[0]
    lens = np.ascontiguousarray(seq_lens, np.int32)
    pt = None if page_table is None else np.ascontiguousarray(page_table, np.int32)
    out = np.zeros((B, fmt.num_q_heads, fmt.head_dim), np.float64)
    rc = lib().orc_decode_attention_folded(ctypes.byref(fmt), _p(q), *[_p(c) for c in cache],
                                           _p(lens), _p(pt),
                                           ctypes.c_int(0 if pt is None else pt.shape[1]),
                                           ctypes.c_int(B), ctypes.c_int(max_len),
                                           ctypes.c_double(scale), ctypes.c_int(1 if bug else 0),
                                           _p(out), ctypes.c_int(_threads(threads)))
    if rc != 0:
        raise ValueError("oracle: unsupported format")
    return out


def decode_attention_bf16(q_bf16, k_bf16, v_bf16, seq_lens, max_len, scale, num_kv_heads,
                          page_size=0, page_table=None, units=None, threads=None):
    """[B][Hq][D] fp64 attention over an unquantised bf16 cache."""
    q = np.ascontiguousarray(q_bf16, np.uint16)
    B, Hq, D = q.shape
    k = np.ascontiguousarray(k_bf16, np.uint16)
    v = np.ascontiguousarray(v_bf16, np.uint16)
    lens = np.ascontiguousarray(seq_lens, np.int32)
    pt = None if page_table is None else np.ascontiguousarray(page_table, np.int32)
    u = None if units is None else np.ascontiguousarray(np.asarray(units, np.int32).reshape(-1, 2))
    out = np.zeros((B, Hq, D), np.float64)
    rc = lib().orc_decode_attention_bf16(ctypes.c_int(num_kv_heads), ctypes.c_int(Hq),
                                         ctypes.c_int(D), ctypes.c_int(page_size), _p(q), _p(k),
                                         _p(v), _p(lens), _p(pt),
                                         ctypes.c_int(0 if pt is None else pt.shape[1]),
                                         ctypes.c_int(B), ctypes.c_int(max_len),
                                         ctypes.c_double(scale), _p(u),
                                         ctypes.c_int(0 if u is None else u.shape[0]), _p(out),
                                         ctypes.c_int(_threads(threads)))
    if rc != 0:
        raise ValueError("oracle: bad arguments")
    return out


def _bf16_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def decode_attention_window(fmt, q_bf16, cache, k_win_bf16, v_win_bf16, seq_lens, max_len, scale,
                            page_table=None):
    """[B][Hq][D] fp64 attention over the tokens of a cache filled by appends:
    tokens [0, Lq) dequantised from the packed cache (Lq = L rounded down to a
    multiple of 128, whole groups only), then tokens [Lq, L) from the bf16
    residual window (token t in row t % 128 of [B][Hkv][128][D]). A plain
    composition of dequantize_unit and attention_f64."""
    q = _bf16_to_f64(q_bf16)
    B, Hq, D = q.shape
    H = fmt.num_kv_heads
    R = Hq // H
    out = np.zeros((B, Hq, D), np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        Lq = L - L % 128
        for h in range(H):
            kh = np.concatenate([dequantize_unit(fmt, "k", cache, b, h, Lq, max_len, page_table),
                                 _bf16_to_f64(k_win_bf16[b, h, :L - Lq])])
            vh = np.concatenate([dequantize_unit(fmt, "v", cache, b, h, Lq, max_len, page_table),
                                 _bf16_to_f64(v_win_bf16[b, h, :L - Lq])])
            out[b, h * R:(h + 1) * R] = attention_f64(q[b, h * R:(h + 1) * R], kh, vh, scale)
    return out
