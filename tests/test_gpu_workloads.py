"""GPU parity at the full sizes of the named workloads, on sampled units the
oracle recomputes one by one, plus the bf16 baseline kernel.

- headline: B=128 x 32768 tokens, INT4 and INT2 (both fold pairings for INT2),
  and token-wise K and V in 64- / 32-channel groups;
- the headline's 8-way tensor-parallel share: one KV head, 4 query heads;
- paged long context: 64 sequences, log-uniform lengths in [1K, 128K], 64-token
  pages scattered over one pool, four layers INT4, INT2, INT4, INT2 run back to
  back on one stream;
- bf16 decode (contiguous and paged) against the oracle's fp64 attention over
  the same bf16 values."""
import math

import numpy as np
import pytest

import oracle
import synth
from kvq_testlib import (MAX_ABS_TOL, REL_L2_TOL, SCALE, gpu_format, group_of, max_abs,
                         pack_rowwise, rel_l2, unit_host_cache)

pytestmark = pytest.mark.gpu


def _decode(w, fmt, cache, table=None, fp8_qk=False, num_splits=0):
    import torch
    import bit_quantized_kv_int2_amd as kvq
    dev = cache[0].device
    q = torch.from_numpy(w.q_bf16().view(np.int16)).to(dev).view(torch.bfloat16)
    lens = torch.tensor(w.seq_lens, dtype=torch.int32, device=dev)
    pt = None if table is None else torch.from_numpy(table).to(dev)
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    kvq.decode_attention_quant(fmt, q, cache, lens, w.max_len, SCALE, out, page_table=pt,
                               fp8_qk=fp8_qk, num_splits=num_splits)
    return out


def _check_units(w, cache, out, units, table=None, num_pages=0, label=""):
    fmt_o = oracle.fmt_of(w, group_of(w))
    q = w.q_bf16()
    got_all, ref_all = [], []
    pool = unit_host_cache(w, fmt_o, cache, 0, table, num_pages) if table is not None else None
    for b in dict.fromkeys(b for b, _ in units):  # one oracle call per sequence, in order
        heads = [h for bb, h in units if bb == b]
        hc = pool if pool is not None else unit_host_cache(w, fmt_o, cache, b)
        if table is None:
            ref = oracle.decode_attention(fmt_o, q[b:b + 1], hc, [w.seq_lens[b]], w.max_len, SCALE,
                                          units=[(0, h) for h in heads])[0]
        else:
            lens = np.zeros(w.batch, np.int32)
            lens[b] = w.seq_lens[b]
            ref = oracle.decode_attention(fmt_o, q, hc, lens, w.max_len, SCALE, page_table=table,
                                          units=[(b, h) for h in heads])[b]
        for h in heads:
            got_all.append(out[b, 4 * h:4 * h + 4].double().cpu().numpy())
            ref_all.append(ref[4 * h:4 * h + 4])
    got_all, ref_all = np.concatenate(got_all), np.concatenate(ref_all)
    e2, ea = rel_l2(got_all, ref_all), max_abs(got_all, ref_all)
    print(f"{label}: {len(units)} units rel_l2={e2:.3e} max_abs={ea:.3e}", flush=True)
    assert np.isfinite(got_all).all()
    assert e2 <= REL_L2_TOL and ea <= MAX_ABS_TOL, (label, e2, ea)


# whole batch rows spread over the batch: every KV head of each
HEADLINE_ROWS = [0, 17, 37, 55, 64, 90, 111, 127]


@pytest.mark.parametrize("bits,k_axis,v_axis", [(4, "channel", "token"), (2, "channel", "token"),
                                                (2, "token", "channel"), (4, "token", "channel")])
def test_headline_sampled(bits, k_axis, v_axis):
    """The headline size in the launch configuration the benchmark times (the
    auto plan: one split per (sequence, KV head)): 8 whole batch rows x 8 KV
    heads (256 query heads) against the oracle, rel-L2 and max-abs over all of
    them; and the packed bytes of one row against the oracle's pack."""
    w = synth.headline(bits, k_axis, v_axis)
    fmt = gpu_format(w)
    cache = pack_rowwise(w, fmt)
    out = _decode(w, fmt, cache)
    units = [(b, h) for b in HEADLINE_ROWS for h in range(w.num_kv_heads)]
    _check_units(w, cache, out, units, label=w.name)
    # packed bytes of a sampled row equal the oracle's pack of the same values
    b = 37
    k = np.stack([w.kv_unit("k", b, h) for h in range(w.num_kv_heads)])[None]
    v = np.stack([w.kv_unit("v", b, h) for h in range(w.num_kv_heads)])[None]
    ref = oracle.quantize_pack(oracle.fmt_of(w), k, v, [w.max_len])
    got = unit_host_cache(w, oracle.fmt_of(w), cache, b)
    for g, o in zip(got, ref):
        assert np.array_equal(np.ascontiguousarray(g).view(np.uint8), np.ascontiguousarray(o).view(np.uint8))


def test_headline_int2_every_unit():
    """The INT2 headline (K channel-wise, V token-wise) as the benchmark times
    it, every one of its 128 x 8 (sequence, KV head) units against the oracle:
    rel-L2 and max-abs over the whole 128 x 32 x 128 output."""
    import os
    import bit_quantized_kv_int2_amd as kvq
    w = synth.headline(2)
    fmt = gpu_format(w)
    cache = pack_rowwise(w, fmt)
    out = _decode(w, fmt, cache).double().cpu().numpy()
    fmt_o = oracle.fmt_of(w)
    row = kvq.kvq_cache_sizes(fmt, 1, w.max_len)
    host = [c.cpu().numpy() for c in cache]
    threads = min(16, os.cpu_count() or 1)
    q = w.q_bf16()
    step = 32
    for b0 in range(0, w.batch, step):  # 32 rows per oracle call, ~0.6 GB of host cache
        shapes = oracle.cache_shapes(fmt_o, step, w.max_len)
        hc = [x[b0 * n:(b0 + step) * n][:int(np.prod(sh)) * np.dtype(dt).itemsize].view(dt).reshape(sh)
              for x, n, (dt, sh) in zip(host, row, shapes)]
        ref = oracle.decode_attention(fmt_o, q[b0:b0 + step], hc, w.seq_lens[b0:b0 + step],
                                      w.max_len, SCALE, threads=threads)
        got = out[b0:b0 + step]
        e2, ea = rel_l2(got, ref), max_abs(got, ref)
        print(f"rows {b0}..{b0 + step - 1}: rel_l2={e2:.3e} max_abs={ea:.3e}", flush=True)
        assert np.isfinite(got).all()
        assert e2 <= REL_L2_TOL and ea <= MAX_ABS_TOL, (b0, e2, ea)


@pytest.mark.parametrize("bits", [2, 4])
def test_headline_sampled_fp8(bits):
    """The fp8-operand q.K^T variant at the full headline size (its own bound:
    the same gate), on the same sampled units."""
    w = synth.headline(bits)
    fmt = gpu_format(w)
    cache = pack_rowwise(w, fmt)
    out = _decode(w, fmt, cache, fp8_qk=True)
    _check_units(w, cache, out, [(0, 0), (37, 5), (64, 3), (127, 7)], label=w.name + "_fp8")


@pytest.mark.parametrize("bits,group", [(2, 64), (4, 32)])
def test_headline_token_groups_sampled(bits, group):
    """Token-wise K and V with 64 / 32 channels per (s, z) pair at the headline
    size: the per-group kernel at its tightest register budgets (INT2 with two
    groups per token at 4 work-groups per CU, INT4 with four at 2)."""
    import dataclasses
    base = synth.headline(bits, "token", "token")
    w = dataclasses.replace(base, name=f"{base.name}_g{group}", extra={"group": group})
    fmt = gpu_format(w)
    cache = pack_rowwise(w, fmt)
    out = _decode(w, fmt, cache)
    _check_units(w, cache, out, [(0, 0), (37, 5), (64, 3), (127, 7)], label=w.name)


@pytest.mark.parametrize("bits", [2, 4])
def test_tp8_share_sampled(bits):
    """One KV head per sequence (an 8-way tensor-parallel share of the headline):
    128 units only, so the automatic plan splits every sequence and the
    log-sum-exp combine runs at this real shape."""
    import bit_quantized_kv_int2_amd as kvq
    w = synth.tp8_share(bits)
    fmt = gpu_format(w)
    assert kvq.kvq_plan_splits(fmt, w.batch, w.max_len) > 1
    cache = pack_rowwise(w, fmt)
    out = _decode(w, fmt, cache)
    _check_units(w, cache, out, [(0, 0), (45, 0), (90, 0), (127, 0)], label=w.name)


def test_paged_long_context_four_layers():
    import torch
    layers = [synth.paged_long(layer) for layer in range(4)]
    lens = layers[0].seq_lens
    table, num_pages = synth.build_page_table(lens, 64, seed=5)
    caches = []
    for w in layers:
        caches.append(pack_rowwise(w, gpu_format(w), table, num_pages))
    # four layers back to back on one stream
    outs = [_decode(w, gpu_format(w), c, table) for w, c in zip(layers, caches)]
    torch.cuda.synchronize()
    order = np.argsort(lens)
    sample = [int(order[0]), int(order[len(order) // 2]), int(order[-1])]
    for li, (w, c, o) in enumerate(zip(layers, caches, outs)):
        units = [(b, (3 * b + li) % w.num_kv_heads) for b in sample]
        _check_units(w, c, o, units, table, num_pages, label=f"paged layer {li} int{w.bits}")
    # the splits planned for these known lengths (what the benchmark runs): many
    # more splits, an odd-padded grid, the combine over them
    import bit_quantized_kv_int2_amd as kvq
    for li in (0, 1):
        w, c = layers[li], caches[li]
        fmt = gpu_format(w)
        ns = kvq.kvq_plan_splits_for_lengths(fmt, lens, w.max_len)
        assert ns > kvq.kvq_plan_splits(fmt, w.batch, w.max_len)
        o = _decode(w, fmt, c, table, num_splits=ns)
        units = [(b, (5 * b + li) % w.num_kv_heads) for b in sample]
        _check_units(w, c, o, units, table, num_pages, label=f"paged layer {li} int{w.bits}, {ns} splits")
        # the fp8 / fp4-operand variant on the same pages and splits (its bound: the same gate)
        o8 = _decode(w, fmt, c, table, fp8_qk=True, num_splits=ns)
        _check_units(w, c, o8, units, table, num_pages,
                     label=f"paged layer {li} int{w.bits}, {ns} splits, fp8 operands")


@pytest.mark.parametrize("paged", [False, True])
def test_bf16_decode_vs_oracle(paged):
    import torch
    import bit_quantized_kv_int2_amd as kvq
    lens = [3000, 1, 0, 129, 2048, 700]
    w = synth.Workload("bf16", len(lens), 2, 8, 128, lens, 4, seed=71, outliers=True)
    k = w.kv_all("k")
    v = w.kv_all("v")
    kb = synth.f32_to_bf16_bits(k)
    vb = synth.f32_to_bf16_bits(v)
    q = w.q_bf16()
    table = None
    if paged:
        table, num_pages = synth.build_page_table(lens, 64, seed=3)
        pool_k = np.zeros((num_pages, 2, 64, 128), np.uint16)
        pool_v = np.zeros_like(pool_k)
        for b, L in enumerate(lens):
            for p in range((L + 63) // 64):
                n = min(64, L - 64 * p)
                pool_k[table[b, p], :, :n] = kb[b, :, 64 * p:64 * p + n]
                pool_v[table[b, p], :, :n] = vb[b, :, 64 * p:64 * p + n]
        kd, vd = pool_k, pool_v
    else:
        kd, vd = kb, vb
    fmt = kvq.make_format(4, "channel", "token", 2, page_size=64 if paged else 0)
    dev = "cuda"
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    out = torch.empty((w.batch, 8, 128), dtype=torch.float32, device=dev)
    kvq.decode_attention_bf16(fmt, to(q), to(kd), to(vd),
                              torch.tensor(lens, dtype=torch.int32, device=dev), w.max_len, SCALE,
                              out, page_table=None if table is None else torch.from_numpy(table).to(dev))
    got = out.double().cpu().numpy()
    ref = oracle.decode_attention_bf16(q, kb, vb, lens, w.max_len, SCALE, 2)
    e2, ea = rel_l2(got, ref), max_abs(got, ref)
    print(f"bf16 paged={paged}: rel_l2={e2:.3e} max_abs={ea:.3e}")
    assert e2 <= REL_L2_TOL and ea <= MAX_ABS_TOL
    assert not got[2].any()
