"""GPU: decode-time append into a bf16 residual window with quantise-on-write
of completed 128-token groups, and the decode over cache + window, against
the oracle (through the C ABI).

The cache after the appends must equal, byte for byte, the oracle's
quantise + pack of the same bf16-rounded values over the whole groups; the
window must hold the remaining tokens' bf16 bits; the decode must be within
rel-L2 4e-3 / max-abs 2e-2 of the oracle's fp64 attention over dequantised
whole groups followed by the window's bf16 tokens."""
import numpy as np
import pytest

import oracle
import synth
from kvq_testlib import (MAX_ABS_TOL, REL_L2_TOL, SCALE, cache_bytes_equal, gpu_format, max_abs,
                         rel_l2)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("bits,k_axis,v_axis,paged,group", [(2, "channel", "token", False, 128),
                                                            (4, "channel", "token", True, 128),
                                                            (2, "token", "channel", False, 128),
                                                            (4, "channel", "channel", False, 128),
                                                            (2, "token", "token", True, 128),
                                                            (4, "token", "token", False, 32),
                                                            (2, "token", "token", True, 64),
                                                            (2, "token", "token", False, 32)])
def test_append_then_window_decode(bits, k_axis, v_axis, paged, group):
    import torch
    import bit_quantized_kv_int2_amd as kvq
    B, H, Lmax = 3, 2, 400
    start = [128, 0, 256]   # whole groups packed in bulk first
    total = [300, 130, 383]  # final lengths (window 44, 2, 127 tokens)
    w = synth.Workload("append", B, H, 4 * H, 128, [Lmax] * B, bits, k_axis, v_axis, seed=81,
                       outliers=True, page_size=64 if paged else 0, extra={"group": group})
    kb = synth.f32_to_bf16_bits(w.kv_all("k"))  # the appended tokens are bf16
    vb = synth.f32_to_bf16_bits(w.kv_all("v"))
    kr = synth.bf16_bits_to_f32(kb)
    vr = synth.bf16_bits_to_f32(vb)
    table, num_pages = (None, 0)
    if paged:
        table, num_pages = synth.build_page_table([Lmax] * B, 64, 5)
    dev = "cuda"
    fmt = gpu_format(w)
    cache = kvq.cache_tensors(fmt, B, Lmax, num_pages, device=dev)
    tdev = None if table is None else torch.from_numpy(table).to(dev)
    kvq.kv_quantize_pack(fmt, torch.from_numpy(kr).to(dev), torch.from_numpy(vr).to(dev),
                         torch.tensor(start, dtype=torch.int32, device=dev), cache, page_table=tdev,
                         max_len=Lmax)
    kwin, vwin = kvq.window_tensors(fmt, B, device=dev)
    kbd = torch.from_numpy(kb.view(np.int16)).to(dev)
    vbd = torch.from_numpy(vb.view(np.int16)).to(dev)
    lens = list(start)
    while any(lens[b] < total[b] for b in range(B)):
        idx = [lens[b] if lens[b] < total[b] else 0 for b in range(B)]
        pos = [lens[b] if lens[b] < total[b] else Lmax for b in range(B)]  # Lmax: leave untouched
        k_new = torch.stack([kbd[b, :, idx[b]] for b in range(B)]).contiguous()
        v_new = torch.stack([vbd[b, :, idx[b]] for b in range(B)]).contiguous()
        kvq.kv_append(fmt, k_new, v_new, torch.tensor(pos, dtype=torch.int32, device=dev), cache,
                      kwin, vwin, Lmax, page_table=tdev)
        lens = [min(lens[b] + 1, total[b]) if lens[b] < total[b] else lens[b] for b in range(B)]
    torch.cuda.synchronize()

    # the cache holds exactly the whole groups, as the bulk rule packs them
    lq = [L - L % 128 for L in total]
    fo = oracle.fmt_of(w, group)
    orc_cache = oracle.quantize_pack(fo, kr, vr, np.asarray(lq, np.int32), page_table=table,
                                     num_pages=num_pages)
    ok, msg = cache_bytes_equal([c.cpu().numpy() for c in cache], orc_cache)
    assert ok, msg
    # the window holds the bf16 bits of the tokens past the last whole group
    kwh = kwin.cpu().view(torch.int16).numpy().view(np.uint16)
    vwh = vwin.cpu().view(torch.int16).numpy().view(np.uint16)
    for b in range(B):
        for t in range(lq[b], total[b]):
            assert np.array_equal(kwh[b, :, t % 128], kb[b, :, t]), (b, t)
            assert np.array_equal(vwh[b, :, t % 128], vb[b, :, t]), (b, t)

    q = w.q_bf16()
    qd = torch.from_numpy(q.view(np.int16)).to(dev).view(torch.bfloat16)
    ref = oracle.decode_attention_window(fo, q, orc_cache, kwh, vwh, total, Lmax, SCALE,
                                         page_table=table)
    lens_d = torch.tensor(total, dtype=torch.int32, device=dev)
    for ns in (1, 2, 0):
        out = torch.empty((B, 4 * H, 128), dtype=torch.float32, device=dev)
        kvq.decode_attention_quant_window(fmt, qd, cache, kwin, vwin, lens_d, Lmax, SCALE, out,
                                          page_table=tdev, num_splits=ns)
        torch.cuda.synchronize()
        o = out.cpu().numpy().astype(np.float64)
        e2, ea = rel_l2(o, ref), max_abs(o, ref)
        print(f"append int{bits} {k_axis[0]}{v_axis[0]} G{group} paged={paged} splits {ns}: "
              f"rel_l2={e2:.3e} max_abs={ea:.3e}")
        assert np.isfinite(o).all()
        assert e2 <= REL_L2_TOL and ea <= MAX_ABS_TOL, (ns, e2, ea)
