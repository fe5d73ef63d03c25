"""GPU parity of the fp8-operand variant (decode_attention_quant_fp8: q.K^T
and P.V on E4M3 / E2M1 operands, for every pairing of K and V groups)
against the fp64 oracle, on the same cases as the fp16-operand path.

Its stated bound is the same gate (rel-L2 <= 4e-3, max-abs <= 2e-2 over each
whole output tensor); the query and the probabilities carry at least 8
significant bits (E4M3 hi + lo / 16; the query exactly for token-wise K), and
the variant is also compared with the fp16-operand path on the same cache."""
import numpy as np
import pytest

import synth
from kvq_testlib import (MAX_ABS_TOL, REL_L2_TOL, GpuRun, Inputs, max_abs, oracle_attention,
                         oracle_pack, rel_l2)

pytestmark = pytest.mark.gpu


def _check(inp, run, label, num_splits=0):
    ref = oracle_attention(inp, oracle_pack(inp))
    o8 = run.decode(num_splits=num_splits, fp8_qk=True)
    o16 = run.decode(num_splits=num_splits)
    e2, ea = rel_l2(o8, ref), max_abs(o8, ref)
    d = rel_l2(o8, o16)
    print(f"{label}: fp8 rel_l2={e2:.3e} max_abs={ea:.3e} (fp16 path {rel_l2(o16, ref):.3e}); "
          f"fp8 vs fp16 {d:.3e}", flush=True)
    assert np.isfinite(o8).all()
    assert e2 <= REL_L2_TOL and ea <= MAX_ABS_TOL, (label, e2, ea)
    return o8, o16, ref


def test_fp8_tiny_int4():
    w = synth.tiny_int4()
    inp = Inputs(w)
    _check(inp, GpuRun(inp), "tiny_int4")


@pytest.mark.parametrize("k_axis,v_axis", [("channel", "token"), ("token", "channel"),
                                           ("channel", "channel"), ("token", "token")])
def test_fp8_mid_int2_all_pairings(k_axis, v_axis):
    w = synth.mid_int2(k_axis, v_axis)
    inp = Inputs(w)
    _check(inp, GpuRun(inp), w.name)


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("k_axis,v_axis", [("channel", "token"), ("token", "channel")])
def test_fp8_ragged_and_constant_groups(bits, k_axis, v_axis):
    lens = [1, 7, 127, 128, 129, 0, 1000, 2047, 2048, 4001]
    w = synth.Workload("ragged8", len(lens), 2, 8, 128, lens, bits, k_axis, v_axis, seed=33,
                       outliers=True)
    inp = Inputs(w)
    inp.k[6, 0, :, 5] = 0.75          # a constant K channel (s = 0 in every channel-wise group)
    inp.k[9, 1, 10, :] = -1.25        # a constant K token
    inp.k[8, 1, 0:128, 77] = 3.0      # one constant channel-wise group
    o8, _, _ = _check(inp, GpuRun(inp), f"ragged_int{bits}_{k_axis[0]}{v_axis[0]}")
    assert not o8[5].any()


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("v_axis", ["token", "channel"])
def test_fp8_splits_and_paging(bits, v_axis):
    lens = [3000, 64, 1, 700, 129]
    w = synth.Workload("paged8", len(lens), 2, 8, 128, lens, bits, "channel", v_axis, seed=63,
                       outliers=True)
    inp = Inputs(w)
    run = GpuRun(inp)
    for ns in (1, 3, 0):
        _check(inp, run, f"splits{ns}_int{bits}_{v_axis}_v", num_splits=ns)
    w_p = synth.Workload("paged8", len(lens), 2, 8, 128, lens, bits, "channel", v_axis, seed=63,
                         outliers=True, page_size=64)
    inp_p = Inputs(w_p)
    run_p = GpuRun(inp_p)
    # paging changes addressing only: the same bits as the contiguous cache
    assert np.array_equal(run_p.decode(fp8_qk=True), run.decode(fp8_qk=True))


@pytest.mark.parametrize("bits", [2, 4])
def test_fp8_channel_wise_v_multi_chunk(bits):
    """Channel-wise V on fp8 P.V operands across 2048-token chunks: each
    64-token iteration's products are folded with its group's (sigma, rho)
    before they reach the accumulators, including groups with larger V
    ranges later in the split and constant (s = 0) groups."""
    w = synth.Workload("chunks8", 2, 1, 4, 128, [6500, 4100], bits, "token", "channel", seed=73,
                       outliers=True)
    inp = Inputs(w)
    inp.v[0, 0, 5000:5100, :] *= 40.0      # larger V scales in sequence 0's third chunk
    inp.v[1, 0, 2100:2230, 3] += 90.0      # one large V channel in sequence 1's second chunk
    inp.v[1, 0, 256:384, 17] = 0.5         # a constant channel-wise V group (s = 0)
    run = GpuRun(inp)
    for ns in (1, 2, 0):
        _check(inp, run, f"chunks_int{bits}_tc_splits{ns}", num_splits=ns)


@pytest.mark.parametrize("v_axis", ["token", "channel"])
def test_fp8_bf16_output(v_axis):
    """bf16 output of the fp8 / fp4-operand variant: the gate holds after the
    output rounding too, and the rows equal the fp32 output rounded."""
    import torch
    w = synth.mid_int2("channel", v_axis)
    inp = Inputs(w)
    run = GpuRun(inp)
    ref = oracle_attention(inp, oracle_pack(inp))
    ob = run.decode(out_dtype=torch.bfloat16, fp8_qk=True)
    of = run.decode(fp8_qk=True)
    assert rel_l2(ob, ref) <= REL_L2_TOL and max_abs(ob, ref) <= MAX_ABS_TOL
    rounded = torch.from_numpy(of.astype(np.float32)).to(torch.bfloat16).float().numpy()
    assert np.array_equal(ob.astype(np.float32), rounded)


def test_fp8_rejects_small_groups():
    import torch
    import bit_quantized_kv_int2_amd as kvq
    w = synth.Workload("g32", 1, 1, 4, 128, [256], 2, "token", "token", seed=5)
    w.extra["group"] = 32
    inp = Inputs(w)
    run = GpuRun(inp)
    with pytest.raises(kvq.KvqError):
        run.decode(fp8_qk=True)
    torch.cuda.synchronize()
