"""Shared helpers for the tests: run a synthetic workload through the GPU
library and through the CPU oracle on the same seeded inputs."""
from __future__ import annotations

import math
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

REL_L2_TOL = 4e-3
MAX_ABS_TOL = 2e-2
SCALE = 1.0 / math.sqrt(128.0)


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a - b))


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)))) if np.size(a) else 0.0


def group_of(w):
    """Group size of a workload (128 unless the workload sets extra['group'])."""
    return int(w.extra.get("group", 128))


def gpu_format(w):
    import bit_quantized_kv_int2_amd as kvq
    return kvq.make_format(w.bits, w.k_axis, w.v_axis, w.num_kv_heads, page_size=w.page_size,
                           group=group_of(w))


class Inputs:
    """Host copies of one workload's inputs (small workloads only)."""

    def __init__(self, w, page_seed=9):
        self.w = w
        self.k = w.kv_all("k")
        self.v = w.kv_all("v")
        self.q = w.q_bf16()
        self.lens = np.asarray(w.seq_lens, np.int32)
        self.table, self.num_pages = (None, 0)
        if w.page_size:
            self.table, self.num_pages = synth.build_page_table(w.seq_lens, w.page_size, page_seed)


def oracle_pack(inp: Inputs):
    w = inp.w
    return oracle.quantize_pack(oracle.fmt_of(w, group_of(w)), inp.k, inp.v, inp.lens,
                                page_table=inp.table,
                                num_pages=inp.num_pages)


def oracle_attention(inp: Inputs, cache, units=None):
    w = inp.w
    return oracle.decode_attention(oracle.fmt_of(w, group_of(w)), inp.q, cache, inp.lens, w.max_len, SCALE,
                                   page_table=inp.table, units=units)


class GpuRun:
    """Device tensors for one workload, packed by the library."""

    def __init__(self, inp: Inputs, device="cuda"):
        import torch
        import bit_quantized_kv_int2_amd as kvq
        self.kvq = kvq
        w = inp.w
        self.inp = inp
        self.fmt = gpu_format(w)
        self.k = torch.from_numpy(inp.k).to(device)
        self.v = torch.from_numpy(inp.v).to(device)
        self.q = torch.from_numpy(inp.q.view(np.int16)).to(device).view(torch.bfloat16)
        self.lens = torch.from_numpy(inp.lens).to(device)
        self.table = None if inp.table is None else torch.from_numpy(inp.table).to(device)
        self.cache = kvq.cache_tensors(self.fmt, w.batch, w.max_len, inp.num_pages, device=device)
        kvq.kv_quantize_pack(self.fmt, self.k, self.v, self.lens, self.cache, self.table,
                             max_len=w.max_len)

    def cache_host(self):
        return [c.cpu().numpy() for c in self.cache]

    def decode(self, num_splits=0, out_dtype=None, fp8_qk=False):
        import torch
        w = self.inp.w
        out = torch.empty((w.batch, w.num_q_heads, w.head_dim), device=self.q.device,
                          dtype=out_dtype or torch.float32)
        self.kvq.decode_attention_quant(self.fmt, self.q, self.cache, self.lens, w.max_len, SCALE,
                                        out, page_table=self.table, num_splits=num_splits,
                                        fp8_qk=fp8_qk)
        torch.cuda.synchronize()
        return out.float().cpu().numpy().astype(np.float64)


def cache_bytes_equal(gpu_cache, orc_cache):
    """Compare the library's packed buffers with the oracle's arrays byte for byte."""
    for i, (g, o) in enumerate(zip(gpu_cache, orc_cache)):
        ob = np.ascontiguousarray(o).view(np.uint8).ravel()
        gb = np.asarray(g).ravel()[:ob.size]
        if not np.array_equal(gb, ob):
            bad = np.nonzero(gb != ob)[0]
            return False, f"array {i}: {bad.size} bytes differ, first at {bad[:8]}"
    return True, ""


def pack_rowwise(w, fmt, table=None, num_pages=0, device="cuda", log=None):
    """Pack a large workload one sequence at a time (host draw -> GPU pack),
    without holding the whole fp32 K/V anywhere. Returns the cache tensors."""
    import torch
    import bit_quantized_kv_int2_amd as kvq
    H, D = w.num_kv_heads, w.head_dim
    L = w.max_len
    cache = kvq.cache_tensors(fmt, w.batch, L, num_pages, device=device)
    offs = w.outlier_offsets()
    kh = np.empty((H, L, D), np.float32)
    vh = np.empty((H, L, D), np.float32)
    for b in range(w.batch):
        Lb = int(w.seq_lens[b])
        if Lb == 0:
            continue
        w.kv_row("k", b, length=Lb, offsets=offs, out=kh[:, :Lb])
        w.kv_row("v", b, length=Lb, out=vh[:, :Lb])
        kd = torch.from_numpy(np.ascontiguousarray(kh[:, :Lb])).to(device)[None]
        vd = torch.from_numpy(np.ascontiguousarray(vh[:, :Lb])).to(device)[None]
        lens = torch.tensor([Lb], dtype=torch.int32, device=device)
        if table is None:
            # contiguous rows are laid out for max_len tokens: every sequence full length
            assert Lb == L, "row-wise contiguous packing needs equal lengths"
            sizes = kvq.kvq_cache_sizes(fmt, 1, L)
            rc = [c[b * n:(b + 1) * n] for c, n in zip(cache, sizes)]
            kvq.kv_quantize_pack(fmt, kd, vd, lens, rc, max_len=Lb)
        else:
            pt = torch.from_numpy(np.ascontiguousarray(table[b:b + 1])).to(device)
            kvq.kv_quantize_pack(fmt, kd, vd, lens, cache, page_table=pt, max_len=Lb)
        if log and b % 16 == 15:
            torch.cuda.synchronize()
            log(f"packed {b + 1}/{w.batch}")
    torch.cuda.synchronize()
    return cache


def unit_host_cache(w, fmt_o, gpu_cache, b, table=None, num_pages=0):
    """Host copy of the packed cache restricted to what the oracle needs for
    sequence b: the contiguous row, or the whole paged pool."""
    import bit_quantized_kv_int2_amd as kvq
    if table is None:
        sizes = kvq.kvq_cache_sizes(gpu_format(w), 1, w.max_len)
        host = [c[b * n:(b + 1) * n].cpu().numpy() for c, n in zip(gpu_cache, sizes)]
        shapes = oracle.cache_shapes(fmt_o, 1, w.max_len)
    else:
        host = [c.cpu().numpy() for c in gpu_cache]
        shapes = oracle.cache_shapes(fmt_o, 0, 0, num_pages)
    return [x[:int(np.prod(sh)) * np.dtype(dt).itemsize].view(dt).reshape(sh)
            for x, (dt, sh) in zip(host, shapes)]
