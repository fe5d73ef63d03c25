"""GPU: decode_attention_quant_noalloc (the entry point that allocates
nothing: its split partials live in the library's per-GPU scratch array)
against decode_attention_quant with a caller workspace, through the C ABI.

Same kernels and split plan, so the outputs must be equal bit for bit; each
is also within the oracle gate. Two calls in a row, the second smaller, so
the second reads the scratch the first left behind in its unused tail; then
a call with one split, which needs no scratch; then two calls with the auto
plan (num_splits = 0), which the decode makes on the device from the lengths."""
import numpy as np
import pytest

import synth
from kvq_testlib import (MAX_ABS_TOL, REL_L2_TOL, SCALE, GpuRun, Inputs, max_abs, oracle_attention,
                         oracle_pack, rel_l2)

pytestmark = pytest.mark.gpu


def _both(run, num_splits):
    import torch
    w = run.inp.w
    outs = []
    for noalloc in (False, True):
        out = torch.full((w.batch, w.num_q_heads, w.head_dim), float("nan"), dtype=torch.float32,
                         device="cuda")
        if noalloc:
            run.kvq.decode_attention_quant_noalloc(run.fmt, run.q, run.cache, run.lens, w.max_len,
                                                   SCALE, out, page_table=run.table,
                                                   num_splits=num_splits)
        else:
            run.kvq.decode_attention_quant(run.fmt, run.q, run.cache, run.lens, w.max_len, SCALE,
                                           out, page_table=run.table, num_splits=num_splits)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy().astype(np.float64))
    return outs


@pytest.mark.parametrize("case", ["large_then_small", "one_split", "auto_plan"])
def test_noalloc_equals_workspace_entry_point(case):
    import bit_quantized_kv_int2_amd as kvq
    if case == "large_then_small":
        calls = [
            (synth.Workload("noalloc_a", 5, 2, 8, 128, [20000, 3000, 0, 17000, 511], 4, "channel",
                            "token", seed=71, outliers=True), 16),
            (synth.Workload("noalloc_b", 2, 1, 4, 128, [900, 5000], 2, "token", "channel", seed=72,
                            page_size=64), 5),
        ]
    elif case == "one_split":
        calls = [(synth.Workload("noalloc_c", 3, 2, 8, 128, [4096, 77, 1000], 2, "channel", "token",
                                 seed=73), 1)]
    else:  # the device-side auto plan on ragged lengths (whole-chunk splits, merged rows)
        calls = [
            (synth.Workload("noalloc_d", 6, 2, 8, 128, [30000, 64, 0, 9000, 2049, 300], 2, "channel",
                            "token", seed=74, outliers=True), 0),
            (synth.Workload("noalloc_e", 3, 1, 4, 128, [7000, 1, 2500], 4, "token", "channel",
                            seed=75, page_size=64), 0),
        ]
    sizes = []
    for w, ns in calls:
        inp = Inputs(w)
        run = GpuRun(inp)
        ref = oracle_attention(inp, oracle_pack(inp))
        need = kvq.kvq_workspace_size(run.fmt, w.batch, w.max_len, ns)
        sizes.append(need)
        assert need <= 32 << 20
        o_ws, o_na = _both(run, ns)
        e2, ea = rel_l2(o_na, ref), max_abs(o_na, ref)
        print(f"noalloc {w.name} splits {ns} scratch {need} B: rel_l2={e2:.3e} max_abs={ea:.3e}")
        assert np.array_equal(o_ws, o_na)
        assert e2 <= REL_L2_TOL and ea <= MAX_ABS_TOL
    if case in ("large_then_small", "auto_plan"):
        assert sizes[1] < sizes[0]
    else:
        assert sizes == [0]
