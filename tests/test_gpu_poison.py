"""GPU: the LDS poison-fill debug build (libkvq_poison.so, built with
KVQ_POISON_LDS: every kernel fills its LDS with all-ones bytes, NaN in
binary16, bf16 and fp32, before first use and at the top of each pass that
reuses it). Pack, decode in every format and split mode, the fp8/fp4-operand
variant, the bf16 decode, append and the window decode must give results
bit-identical to the normal build's: no kernel reads LDS that it did not
write first. The normal build's results are checked against the oracle by
the other GPU tests."""
import contextlib
import os

import numpy as np
import pytest

import synth
from kvq_testlib import SCALE, Inputs, gpu_format

pytestmark = pytest.mark.gpu


@contextlib.contextmanager
def _library(path):
    """Route the binding's calls to the library at path for the block."""
    import bit_quantized_kv_int2_amd as kvq
    saved = kvq._lib, kvq.LIB_PATH
    kvq._lib, kvq.LIB_PATH = None, path
    try:
        yield kvq.lib()
    finally:
        kvq._lib, kvq.LIB_PATH = saved


def _quant_cases():
    lens = [2500, 77, 2048 + 64 + 5]
    for bits in (2, 4):
        for ka, va in [("channel", "token"), ("token", "channel"), ("channel", "channel"),
                       ("token", "token")]:
            yield synth.Workload(f"p{bits}{ka[0]}{va[0]}", 3, 2, 8, 128, lens, bits, ka, va,
                                 seed=101, outliers=True)
    yield synth.Workload("paged2", 3, 2, 8, 128, lens, 2, "channel", "token", seed=102,
                         page_size=64)
    yield synth.Workload("paged4", 3, 2, 8, 128, lens, 4, "token", "channel", seed=103,
                         page_size=64)
    for bits in (2, 4):
        for g in (32, 64):
            yield synth.Workload(f"tg{bits}_{g}", 3, 2, 8, 128, lens, bits, "token", "token",
                                 seed=104, outliers=True, extra={"group": g})
    yield synth.Workload("tg_paged2_32", 3, 2, 8, 128, lens, 2, "token", "token", seed=107,
                         page_size=64, extra={"group": 32})
    yield synth.Workload("tg_paged4_64", 3, 2, 8, 128, lens, 4, "token", "token", seed=108,
                         page_size=64, extra={"group": 64})


def _run_everything():
    """Every kernel on fixed seeded inputs; returns {name: host array}."""
    import torch
    import bit_quantized_kv_int2_amd as kvq
    dev = "cuda"
    res = {}
    for w in _quant_cases():
        inp = Inputs(w)
        fmt = gpu_format(w)
        k, v = torch.from_numpy(inp.k).to(dev), torch.from_numpy(inp.v).to(dev)
        q = torch.from_numpy(inp.q.view(np.int16)).to(dev).view(torch.bfloat16)
        lens = torch.from_numpy(inp.lens).to(dev)
        table = None if inp.table is None else torch.from_numpy(inp.table).to(dev)
        cache = kvq.cache_tensors(fmt, w.batch, w.max_len, inp.num_pages, device=dev)
        for c in cache:
            c.fill_(0x5A)  # bytes the pack does not write stay the same in both runs
        kvq.kv_quantize_pack(fmt, k, v, lens, cache, table, max_len=w.max_len)
        for i, c in enumerate(cache):
            res[f"{w.name} cache {i}"] = c.cpu().numpy()
        modes = [(ns, False) for ns in (1, 3, 0)]
        if w.extra.get("group", 128) == 128:
            modes.append((0, True))
        for ns, fp8 in modes:
            for od in (torch.float32, torch.bfloat16):
                out = torch.empty((w.batch, w.num_q_heads, 128), dtype=od, device=dev)
                kvq.decode_attention_quant(fmt, q, cache, lens, w.max_len, SCALE, out,
                                           page_table=table, num_splits=ns, fp8_qk=fp8)
                res[f"{w.name} decode ns={ns} fp8={fp8} {od}"] = out.float().cpu().numpy()
        out = torch.empty((w.batch, w.num_q_heads, 128), dtype=torch.float32, device=dev)
        kvq.decode_attention_quant_noalloc(fmt, q, cache, lens, w.max_len, SCALE, out,
                                           page_table=table)
        res[f"{w.name} noalloc"] = out.cpu().numpy()
        torch.cuda.synchronize()

    # bf16 decode, contiguous
    lens = [3000, 1, 0, 129, 2048, 700]
    w = synth.Workload("bf16", len(lens), 2, 8, 128, lens, 4, seed=105, outliers=True)
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(
        torch.bfloat16)
    kb, vb = synth.f32_to_bf16_bits(w.kv_all("k")), synth.f32_to_bf16_bits(w.kv_all("v"))
    fmt = kvq.make_format(4, "channel", "token", 2)
    ld = torch.tensor(lens, dtype=torch.int32, device=dev)
    for ns in (1, 0):
        out = torch.empty((w.batch, 8, 128), dtype=torch.float32, device=dev)
        kvq.decode_attention_bf16(fmt, to(w.q_bf16()), to(kb), to(vb), ld, w.max_len, SCALE, out,
                                  num_splits=ns)
        res[f"bf16 ns={ns}"] = out.cpu().numpy()

    # append into the bf16 window with group flushes, then the window decode
    for bits, ka, va, g in [(2, "channel", "token", 128), (4, "token", "channel", 128),
                            (2, "token", "token", 32)]:
        B, H, Lmax = 2, 2, 400
        w = synth.Workload("append", B, H, 8, 128, [Lmax] * B, bits, ka, va, seed=106,
                           outliers=True, extra={"group": g})
        fmt = gpu_format(w)
        kbits = synth.f32_to_bf16_bits(w.kv_all("k"))
        vbits = synth.f32_to_bf16_bits(w.kv_all("v"))
        cache = kvq.cache_tensors(fmt, B, Lmax, device=dev)
        for c in cache:
            c.fill_(0x5A)
        start, total = [128, 0], [300, 130]
        kvq.kv_quantize_pack(fmt, torch.from_numpy(synth.bf16_bits_to_f32(kbits)).to(dev),
                             torch.from_numpy(synth.bf16_bits_to_f32(vbits)).to(dev),
                             torch.tensor(start, dtype=torch.int32, device=dev), cache,
                             max_len=Lmax)
        kwin, vwin = kvq.window_tensors(fmt, B, device=dev)
        kbd = torch.from_numpy(kbits.view(np.int16)).to(dev)
        vbd = torch.from_numpy(vbits.view(np.int16)).to(dev)
        cur = list(start)
        while any(cur[b] < total[b] for b in range(B)):
            idx = [cur[b] if cur[b] < total[b] else 0 for b in range(B)]
            pos = [cur[b] if cur[b] < total[b] else Lmax for b in range(B)]
            k_new = torch.stack([kbd[b, :, idx[b]] for b in range(B)]).contiguous()
            v_new = torch.stack([vbd[b, :, idx[b]] for b in range(B)]).contiguous()
            kvq.kv_append(fmt, k_new, v_new, torch.tensor(pos, dtype=torch.int32, device=dev),
                          cache, kwin, vwin, Lmax)
            cur = [min(c + 1, t) for c, t in zip(cur, total)]
        name = f"append{bits}{ka[0]}{va[0]}G{g}"
        for i, c in enumerate(cache):
            res[f"{name} cache {i}"] = c.cpu().numpy()
        res[f"{name} kwin"] = kwin.cpu().view(torch.int16).numpy()
        res[f"{name} vwin"] = vwin.cpu().view(torch.int16).numpy()
        qd = to(w.q_bf16())
        for ns in (1, 0):
            out = torch.empty((B, 8, 128), dtype=torch.float32, device=dev)
            kvq.decode_attention_quant_window(fmt, qd, cache, kwin, vwin,
                                              torch.tensor(total, dtype=torch.int32, device=dev),
                                              Lmax, SCALE, out, num_splits=ns)
            res[f"{name} window ns={ns}"] = out.cpu().numpy()
    torch.cuda.synchronize()
    return res


def test_poison_build_matches_normal_build():
    import bit_quantized_kv_int2_amd as kvq
    from bit_quantized_kv_int2_amd import build
    if not os.path.exists(build.POISON_LIB):
        pytest.skip("libkvq_poison.so is not built (build.build(poison=True))")
    with _library(build.LIB) as L:
        assert L.kvq_build_flags() == 0
        normal = _run_everything()
    with _library(build.POISON_LIB) as L:
        assert L.kvq_build_flags() == 1  # KVQ_BUILD_POISON_LDS
        poisoned = _run_everything()
    assert kvq.lib().kvq_build_flags() == 0  # the binding is back on the normal build
    assert normal.keys() == poisoned.keys()
    bad = []
    for name, a in normal.items():
        b = poisoned[name]
        if not np.array_equal(a.view(np.uint8), b.view(np.uint8)):
            bad.append(name)
        elif a.dtype.kind == "f":
            assert np.isfinite(a).all(), name
    print(f"{len(normal)} results compared", flush=True)
    assert not bad, f"results differ under the LDS poison fill: {bad}"
