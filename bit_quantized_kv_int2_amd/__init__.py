"""Python binding of libkvq.so: INT2/INT4 affine-folded decode attention on MI355X.

Argument marshalling only. Every step of quantise/pack and decode runs in the
library's HIP kernels; PyTorch supplies device memory and the current stream.
There is no fallback: importing works without the library (so host-side
helpers and tests can report a clear error), but every call that needs it
raises if libkvq.so is missing or no GPU is present.

Names follow the C ABI in include/kvq.h: kv_quantize_pack,
decode_attention_quant, decode_attention_bf16, plus the host-only size and
plan queries.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkvq.so")

TOKEN_WISE, CHANNEL_WISE = 0, 1
OUT_F32, OUT_BF16 = 0, 1
LAYOUT_VERSION = 2
AXES = {"token": TOKEN_WISE, "channel": CHANNEL_WISE, TOKEN_WISE: TOKEN_WISE,
        CHANNEL_WISE: CHANNEL_WISE}

STATUS = {0: "KVQ_OK", 1: "KVQ_ERR_NULL_POINTER", 2: "KVQ_ERR_BAD_FORMAT", 3: "KVQ_ERR_BAD_SHAPE",
          4: "KVQ_ERR_MISALIGNED", 5: "KVQ_ERR_WORKSPACE", 6: "KVQ_ERR_HIP"}


class KvqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        extra = ""
        if status == 6 and _lib is not None:
            extra = f" (hipError_t {_lib.kvq_last_hip_error()})"
        super().__init__(f"{where}: {STATUS.get(status, status)}{extra}")


class Format(ctypes.Structure):
    """kvq_format: bits, k_axis, v_axis, group, head_dim, num_kv_heads,
    num_q_heads, page_size, layout_version."""
    _fields_ = [("bits", ctypes.c_int32), ("k_axis", ctypes.c_int32), ("v_axis", ctypes.c_int32),
                ("group", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("layout_version", ctypes.c_uint32)]


class Cache(ctypes.Structure):
    _fields_ = [("k_codes", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
                ("k_scale_offset", ctypes.c_void_p), ("v_scale_offset", ctypes.c_void_p)]


def make_format(bits, k_axis="channel", v_axis="token", num_kv_heads=1, page_size=0,
                group=128, head_dim=128, num_q_heads=None, layout_version=LAYOUT_VERSION):
    return Format(bits, AXES[k_axis], AXES[v_axis], group, head_dim, num_kv_heads,
                  4 * num_kv_heads if num_q_heads is None else num_q_heads, page_size,
                  layout_version)


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32


def lib():
    """The loaded libkvq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "bit_quantized_kv_int2_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        FP = ctypes.POINTER(Format)
        L.kvq_status_string.restype = ctypes.c_char_p
        L.kvq_status_string.argtypes = [ctypes.c_int]
        L.kvq_last_hip_error.restype = ctypes.c_int32
        L.kvq_debug_inject_hip_error.argtypes = [ctypes.c_int32]
        L.kvq_debug_inject_hip_error.restype = None
        L.kvq_layout_version.restype = ctypes.c_uint32
        L.kvq_build_flags.restype = ctypes.c_uint32
        L.kvq_check_format.argtypes = [FP]
        L.kvq_cache_sizes.argtypes = [FP, _I, _I, _I, ctypes.POINTER(ctypes.c_size_t)]
        L.kvq_plan_splits.argtypes = [FP, _I, _I, ctypes.POINTER(ctypes.c_int32)]
        L.kvq_plan_splits_for_lengths.argtypes = [FP, _I, _I, _P, ctypes.POINTER(ctypes.c_int32)]
        L.kvq_auto_plan.argtypes = [FP, _I, _I, _P] + [ctypes.POINTER(ctypes.c_int32)] * 3
        L.kvq_workspace_size.argtypes = [FP, _I, _I, _I, ctypes.POINTER(ctypes.c_size_t)]
        L.kv_quantize_pack.argtypes = [FP, _P, _P, _P, _P, _I, _I, _I, ctypes.POINTER(Cache), _P]
        L.decode_attention_quant.argtypes = [FP, _P, ctypes.POINTER(Cache), _P, _P, _I, _I, _I,
                                             ctypes.c_float, _P, _I, _I, _P, ctypes.c_size_t, _P]
        L.decode_attention_quant_fp8.argtypes = L.decode_attention_quant.argtypes
        L.decode_attention_quant_noalloc.argtypes = [FP, _P, ctypes.POINTER(Cache), _P, _P, _I, _I,
                                                     _I, ctypes.c_float, _P, _I, _I, _P]
        L.decode_attention_bf16.argtypes = [FP, _P, _P, _P, _P, _P, _I, _I, _I, ctypes.c_float,
                                            _P, _I, _I, _P, ctypes.c_size_t, _P]
        L.kvq_stream_read.argtypes = [_P, ctypes.c_size_t, _P, _P]
        L.kvq_issue_probe.argtypes = [_I, _I, _I, _P, _P]
        L.kv_append.argtypes = [FP, _P, _P, _P, _P, _I, _I, _I, ctypes.POINTER(Cache), _P, _P, _P]
        L.kvq_window_workspace_size.argtypes = [FP, _I, _I, _I, ctypes.POINTER(ctypes.c_size_t)]
        L.decode_attention_quant_window.argtypes = [FP, _P, ctypes.POINTER(Cache), _P, _P, _P, _P,
                                                    _I, _I, _I, ctypes.c_float, _P, _I, _I, _P,
                                                    ctypes.c_size_t, _P]
        for fn in ("kvq_check_format", "kvq_cache_sizes", "kvq_plan_splits",
                   "kvq_plan_splits_for_lengths", "kvq_auto_plan", "kvq_workspace_size",
                   "kv_quantize_pack", "decode_attention_quant", "decode_attention_quant_fp8",
                   "decode_attention_quant_noalloc", "decode_attention_bf16",
                   "kvq_stream_read", "kvq_issue_probe", "kv_append", "kvq_window_workspace_size",
                   "decode_attention_quant_window"):
            getattr(L, fn).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int, where: str):
    if status != 0:
        raise KvqError(status, where)


# ---- host-only queries -----------------------------------------------------

def kvq_debug_inject_hip_error(hip_error: int) -> None:
    """While non-zero, entry points on this thread fail with KVQ_ERR_HIP and
    this hipError_t after their host checks, making no HIP call (0: off)."""
    lib().kvq_debug_inject_hip_error(int(hip_error))


def kvq_check_format(fmt: Format) -> int:
    return lib().kvq_check_format(ctypes.byref(fmt))


def kvq_cache_sizes(fmt: Format, batch: int, max_len: int, num_pages: int = 0):
    out = (ctypes.c_size_t * 4)()
    _check(lib().kvq_cache_sizes(ctypes.byref(fmt), batch, max_len, num_pages, out),
           "kvq_cache_sizes")
    return [int(v) for v in out]


def kvq_plan_splits(fmt: Format, batch: int, max_len: int) -> int:
    n = ctypes.c_int32()
    _check(lib().kvq_plan_splits(ctypes.byref(fmt), batch, max_len, ctypes.byref(n)),
           "kvq_plan_splits")
    return int(n.value)


def kvq_plan_splits_for_lengths(fmt: Format, seq_lens, max_len: int) -> int:
    """num_splits for a batch whose lengths are known on the host (sequence of ints)."""
    import numpy as np
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    n = ctypes.c_int32()
    _check(lib().kvq_plan_splits_for_lengths(ctypes.byref(fmt), int(lens.size), int(max_len),
                                             lens.ctypes.data_as(ctypes.c_void_p),
                                             ctypes.byref(n)), "kvq_plan_splits_for_lengths")
    return int(n.value)


def kvq_auto_plan(fmt: Format, seq_lens, max_len: int):
    """(split_tokens, items, grid) of the quantised decode's auto plan for these
    lengths (host copy of the rule the decode applies on the device)."""
    import numpy as np
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    out = [ctypes.c_int32() for _ in range(3)]
    _check(lib().kvq_auto_plan(ctypes.byref(fmt), int(lens.size), int(max_len),
                               lens.ctypes.data_as(ctypes.c_void_p), *[ctypes.byref(o) for o in out]),
           "kvq_auto_plan")
    return tuple(int(o.value) for o in out)


def kvq_workspace_size(fmt: Format, batch: int, max_len: int, num_splits: int = 0) -> int:
    n = ctypes.c_size_t()
    _check(lib().kvq_workspace_size(ctypes.byref(fmt), batch, max_len, num_splits,
                                    ctypes.byref(n)), "kvq_workspace_size")
    return int(n.value)


# ---- device calls (torch tensors in, results written in place) -----------------

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _require_gpu(*tensors):
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("bit_quantized_kv_int2_amd needs a ROCm GPU; none is visible")
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be device tensors")


def cache_tensors(fmt: Format, batch: int, max_len: int, num_pages: int = 0, device="cuda"):
    """Zero-filled device tensors for one layer's packed cache (uint8 buffers)."""
    import torch
    sizes = kvq_cache_sizes(fmt, batch, max_len, num_pages)
    return [torch.zeros(max(s, 16), dtype=torch.uint8, device=device) for s in sizes]


def workspace_tensor(fmt: Format, batch: int, max_len: int, num_splits: int = 0, device="cuda"):
    """Zero-filled workspace for decode calls: the per-split partials (m, l, O)
    that the combine kernel merges."""
    import torch
    ws = kvq_workspace_size(fmt, batch, max_len, num_splits)
    return torch.zeros(max(ws, 16), dtype=torch.uint8, device=device)


def _cache_struct(cache):
    return Cache(*[c.data_ptr() for c in cache])


def kv_quantize_pack(fmt: Format, k, v, seq_lens, cache, page_table=None, max_len=None,
                     stream=None):
    """Quantise + pack K, V (fp32 [B][Hkv][max_len][D] device tensors) into cache."""
    _require_gpu(k, v, seq_lens, page_table)
    B = k.shape[0]
    max_len = k.shape[2] if max_len is None else max_len
    maxp = 0 if page_table is None else page_table.shape[1]
    cs = _cache_struct(cache)
    _check(lib().kv_quantize_pack(ctypes.byref(fmt), _ptr(k), _ptr(v), _ptr(seq_lens),
                                  _ptr(page_table), maxp, B, max_len, ctypes.byref(cs),
                                  _stream(stream)), "kv_quantize_pack")


def decode_attention_quant(fmt: Format, q, cache, seq_lens, max_len, softmax_scale, out,
                           page_table=None, num_splits=0, workspace=None, stream=None,
                           fp8_qk=False):
    """out[B][Hq][D] (fp32 or bf16 tensor) = decode attention of q (bf16) over cache.
    fp8_qk=True calls decode_attention_quant_fp8 (q.K^T on E4M3 operands)."""
    import torch
    _require_gpu(q, seq_lens, out, page_table)
    B = q.shape[0]
    if workspace is None:
        workspace = workspace_tensor(fmt, B, max_len, num_splits, q.device)
    maxp = 0 if page_table is None else page_table.shape[1]
    od = OUT_BF16 if out.dtype == torch.bfloat16 else OUT_F32
    cs = _cache_struct(cache)
    name = "decode_attention_quant_fp8" if fp8_qk else "decode_attention_quant"
    _check(getattr(lib(), name)(ctypes.byref(fmt), _ptr(q), ctypes.byref(cs),
                                _ptr(seq_lens), _ptr(page_table), maxp, B, max_len,
                                float(softmax_scale), _ptr(out), od, num_splits,
                                _ptr(workspace), workspace.numel(), _stream(stream)), name)
    return out


def decode_attention_quant_noalloc(fmt: Format, q, cache, seq_lens, max_len, softmax_scale, out,
                                   page_table=None, num_splits=0, stream=None):
    """decode_attention_quant without a workspace: the split partials go to
    the library's per-GPU scratch array (no allocation in the call)."""
    import torch
    _require_gpu(q, seq_lens, out, page_table)
    B = q.shape[0]
    maxp = 0 if page_table is None else page_table.shape[1]
    od = OUT_BF16 if out.dtype == torch.bfloat16 else OUT_F32
    cs = _cache_struct(cache)
    _check(lib().decode_attention_quant_noalloc(ctypes.byref(fmt), _ptr(q), ctypes.byref(cs),
                                                _ptr(seq_lens), _ptr(page_table), maxp, B,
                                                max_len, float(softmax_scale), _ptr(out), od,
                                                num_splits, _stream(stream)),
           "decode_attention_quant_noalloc")
    return out


def decode_attention_bf16(fmt: Format, q, k, v, seq_lens, max_len, softmax_scale, out,
                          page_table=None, num_splits=0, workspace=None, stream=None):
    """out[B][Hq][D] = decode attention of q over an unquantised bf16 cache."""
    import torch
    _require_gpu(q, k, v, seq_lens, out, page_table)
    B = q.shape[0]
    if workspace is None:
        workspace = workspace_tensor(fmt, B, max_len, num_splits, q.device)
    maxp = 0 if page_table is None else page_table.shape[1]
    od = OUT_BF16 if out.dtype == torch.bfloat16 else OUT_F32
    _check(lib().decode_attention_bf16(ctypes.byref(fmt), _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(seq_lens), _ptr(page_table), maxp, B, max_len,
                                       float(softmax_scale), _ptr(out), od, num_splits,
                                       _ptr(workspace), workspace.numel(), _stream(stream)),
           "decode_attention_bf16")
    return out


def kvq_window_workspace_size(fmt: Format, batch: int, max_len: int, num_splits: int = 0) -> int:
    n = ctypes.c_size_t()
    _check(lib().kvq_window_workspace_size(ctypes.byref(fmt), batch, max_len, num_splits,
                                           ctypes.byref(n)), "kvq_window_workspace_size")
    return int(n.value)


def window_tensors(fmt: Format, batch: int, device="cuda"):
    """Zero-filled bf16 residual windows (K, V) [batch][Hkv][128][D] for kv_append."""
    import torch
    shape = (batch, fmt.num_kv_heads, 128, fmt.head_dim)
    return (torch.zeros(shape, dtype=torch.bfloat16, device=device),
            torch.zeros(shape, dtype=torch.bfloat16, device=device))


def kv_append(fmt: Format, k_new, v_new, seq_lens, cache, k_window, v_window, max_len,
              page_table=None, stream=None):
    """Append one token per sequence (bf16 [B][Hkv][D]) at index seq_lens[b]."""
    _require_gpu(k_new, v_new, seq_lens, k_window, v_window, page_table)
    B = k_new.shape[0]
    maxp = 0 if page_table is None else page_table.shape[1]
    cs = _cache_struct(cache)
    _check(lib().kv_append(ctypes.byref(fmt), _ptr(k_new), _ptr(v_new), _ptr(seq_lens),
                           _ptr(page_table), maxp, B, max_len, ctypes.byref(cs), _ptr(k_window),
                           _ptr(v_window), _stream(stream)), "kv_append")


def decode_attention_quant_window(fmt: Format, q, cache, k_window, v_window, seq_lens, max_len,
                                  softmax_scale, out, page_table=None, num_splits=0,
                                  workspace=None, stream=None):
    """Decode over whole groups in the packed cache plus the bf16 residual window."""
    import torch
    _require_gpu(q, seq_lens, out, k_window, v_window, page_table)
    B = q.shape[0]
    if workspace is None:
        ws = kvq_window_workspace_size(fmt, B, max_len, num_splits)
        workspace = torch.zeros(max(ws, 16), dtype=torch.uint8, device=q.device)
    maxp = 0 if page_table is None else page_table.shape[1]
    od = OUT_BF16 if out.dtype == torch.bfloat16 else OUT_F32
    cs = _cache_struct(cache)
    _check(lib().decode_attention_quant_window(
        ctypes.byref(fmt), _ptr(q), ctypes.byref(cs), _ptr(k_window), _ptr(v_window),
        _ptr(seq_lens), _ptr(page_table), maxp, B, max_len, float(softmax_scale), _ptr(out), od,
        num_splits, _ptr(workspace), workspace.numel(), _stream(stream)),
        "decode_attention_quant_window")
    return out


def kvq_stream_read(buf, sink, nbytes=None, stream=None):
    """Measurement reference: read nbytes of a device tensor once (128-bit loads)."""
    _require_gpu(buf, sink)
    n = buf.numel() * buf.element_size() if nbytes is None else nbytes
    _check(lib().kvq_stream_read(_ptr(buf), n, _ptr(sink), _stream(stream)), "kvq_stream_read")


def kvq_issue_probe(mode, iters, blocks, out, stream=None):
    """Measurement: matrix-product / vector-instruction overlap probe (modes 0-3); out is a
    float32 device tensor of at least blocks * 256 elements."""
    import torch
    _require_gpu(out)
    if out.dtype != torch.float32 or out.numel() < blocks * 256:
        raise ValueError("kvq_issue_probe: out must be float32 with blocks * 256 elements")
    _check(lib().kvq_issue_probe(int(mode), int(iters), int(blocks), _ptr(out), _stream(stream)),
           "kvq_issue_probe")
