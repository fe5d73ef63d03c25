"""Pins for the CPU oracle against things other than itself.

Each test pins one part of the oracle to an independent fact: numpy's IEEE
binary16 conversion, brute-force search over all codes, hand-worked layout
examples, closed forms of softmax attention, torch's fp64 attention routine,
and the pages' statement that the affine folds reproduce the dequantised
result exactly in exact arithmetic (arXiv abstract; rag-lover.com explainer).
"""
import math

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# --------------------------------------------------------------------------
# binary16 conversion vs numpy
# --------------------------------------------------------------------------

def test_f16_conversion_matches_numpy(orc):
    rng = np.random.default_rng(7)
    vals = [rng.standard_normal(3000).astype(np.float32) * np.float32(10.0) ** rng.integers(-9, 6, 3000)]
    # exact binary16 ties and their neighbours, subnormal range, overflow boundary
    base = np.arange(0, 2048, dtype=np.float64)
    for e in (-26, -25, -24, -20, -14, -10, 0, 5):
        t = ((base + 0.5) * 2.0 ** e).astype(np.float32)
        vals += [t, np.nextafter(t, np.float32(np.inf)), np.nextafter(t, np.float32(0))]
    vals.append(np.array([65504, 65519.99, 65520, 65536, 1e6, 6.1e-5, 5.96e-8, 2.98e-8, 2.99e-8,
                          0.0, -0.0, 1e-40, np.inf, -np.inf], np.float32))
    x = np.concatenate(vals).astype(np.float32)
    x = np.concatenate([x, -x])
    got = orc.f32_to_f16_bits(x)
    want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)
    # and back: exact decode of every binary16 pattern that is finite
    allbits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    fin = np.isfinite(allbits.view(np.float16))
    dec = orc.f16_bits_to_f64(allbits[fin][::37])
    assert np.array_equal(dec, allbits[fin][::37].view(np.float16).astype(np.float64))


# --------------------------------------------------------------------------
# group quantiser
# --------------------------------------------------------------------------

def _f16(v):
    return float(np.float32(v).astype(np.float16))


def test_quantizer_hand_cases(orc):
    # INT2 values exactly on the grid: s = (3-0)/3 = 1, z = 0, codes = values
    x = np.array([0, 1, 2, 3] * 32, np.float32)
    s, z, c = orc.quantize_group(x, 2)
    assert _f16(1.0) == orc.f16_bits_to_f64(s) and orc.f16_bits_to_f64(z) == 0.0
    assert np.array_equal(c, x.astype(np.uint8))
    # ties go to even: 0.5 -> 0, 1.5 -> 2, 2.5 -> 2
    x = np.array([0, 0.5, 1.5, 2.5, 3] + [1.0] * 123, np.float32)
    s, z, c = orc.quantize_group(x, 2)
    assert list(c[:5]) == [0, 0, 2, 2, 3]
    # constant group: s == 0, every code 0, z = the value
    x = np.full(128, 0.3, np.float32)
    s, z, c = orc.quantize_group(x, 4)
    assert s == 0 and z == np.float16(0.3).view(np.uint16) and not c.any()
    # INT4 [-1, 14]: s = 1, z = -1, codes 0 and 15
    x = np.array([-1.0, 14.0] * 64, np.float32)
    s, z, c = orc.quantize_group(x, 4)
    assert orc.f16_bits_to_f64(s) == 1.0 and orc.f16_bits_to_f64(z) == -1.0
    assert list(c[:2]) == [0, 15]
    # s rounds through binary16: range 1/3 per step is not exact
    x = np.linspace(0.0, 1.0, 128).astype(np.float32)
    s, z, c = orc.quantize_group(x, 2)
    assert s == np.float16(np.float32(1.0) / np.float32(3.0)).view(np.uint16)
    # min and max order -0 below +0 (IEEE 754-2019 minimum / maximum), so z
    # does not depend on where the zeros sit in the group
    for vals in ([0.0, -0.0, 1.0], [-0.0, 0.0, 1.0], [1.0, 0.0, -0.0], [1.0, -0.0, 0.0, -0.0]):
        s, z, c = orc.quantize_group(np.array(vals, np.float32), 2)
        assert z == 0x8000 and s == np.float16(1.0 / 3.0).view(np.uint16), vals
    for vals in ([0.0, 0.0, 1.0], [1.0, 0.0]):
        s, z, c = orc.quantize_group(np.array(vals, np.float32), 2)
        assert z == 0x0000, vals
    # a group of zeros of both signs is a constant group: s = 0, z = -0
    s, z, c = orc.quantize_group(np.array([0.0, -0.0, 0.0], np.float32), 4)
    assert s == 0 and z == 0x8000 and not c.any()


@pytest.mark.parametrize("bits", [2, 4])
def test_quantizer_brute_force(orc, bits):
    """Every code is the nearest grid point of the stored (s, z), found by
    trying all 2^b codes, except within rounding distance of a tie."""
    rng = np.random.default_rng(100 + bits)
    qmax = (1 << bits) - 1
    for trial in range(60):
        n = int(rng.integers(1, 130))
        scale = 10.0 ** rng.uniform(-3, 2)
        x = (rng.standard_normal(n) * scale + rng.uniform(-5, 5) * scale).astype(np.float32)
        s, z, c = orc.quantize_group(x, bits)
        S, Z = orc.f16_bits_to_f64(s), orc.f16_bits_to_f64(z)
        assert c.max() <= qmax
        if S == 0:
            assert not c.any()
            continue
        grid = S * np.arange(qmax + 1) + Z
        err = np.abs(x[:, None].astype(np.float64) - grid[None, :])
        best = err.argmin(axis=1)
        t = (x.astype(np.float64) - Z) / S
        near_tie = np.abs(t - np.floor(t) - 0.5) < 1e-4
        ok = (best == c) | near_tie
        assert ok.all(), (trial, x[~ok], c[~ok], best[~ok])
        # reconstruction error bound: half a step plus what fp16 rounding of s, z costs
        s32 = (np.float32(x.max()) - np.float32(x.min())) / np.float32(qmax)
        bound = S / 2 + qmax * abs(S - float(s32)) + abs(Z - float(x.min())) + 1e-6 * scale
        assert np.all(np.abs(x - (S * c + Z)) <= bound)


# --------------------------------------------------------------------------
# packed layout: hand-worked examples
# --------------------------------------------------------------------------

def _grid_data(L, D, bits, transpose=False):
    """Values already on the integer grid 0..qmax with both 0 and qmax in every
    token row and every 128-token channel column, so s = 1, z = 0 and the codes
    equal the values whatever the grouping."""
    qmax = (1 << bits) - 1
    t = np.arange(L)[:, None]
    d = np.arange(D)[None, :]
    x = ((t * 3 + d) % (qmax + 1)).astype(np.float32)
    return x


def _golden(name):
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", name)
    cases = {}
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, val = line.split("=", 1)
        cases[key.strip()] = val.strip()
    return cases


def _slot_tables():
    """Per-bit-width token -> 16-byte slot maps of a 64-token block, read from
    the hand-worked rho lists in the golden file's comments."""
    rho = {4: [0, 2, 4, 6, 1, 3, 5, 7, 8, 10, 12, 14, 9, 11, 13, 15],
           2: [0, 2, 4, 6, 8, 10, 12, 14, 1, 3, 5, 7, 9, 11, 13, 15]}
    return {b: np.array([16 * (u // 16) + r[u % 16] for u in range(64)]) for b, r in rho.items()}


def _unblock_k(blocks, bits):
    """[nblk][64*rowbytes] block-order K bytes -> [nblk*64][rowbytes] token rows."""
    rowb = 128 * bits // 8
    slot = _slot_tables()[bits]
    out = np.empty((blocks.shape[0], 64, rowb), np.uint8)
    for u in range(64):
        for piece in range(rowb // 16):
            p0 = 1024 * piece + 16 * slot[u]
            out[:, u, 16 * piece:16 * piece + 16] = blocks[:, p0:p0 + 16]
    return out.reshape(-1, rowb)


def _unblock_v(blocks, bits):
    """[nblk][(64/tpw)*128] block-order V words -> [nblk*64/tpw][128] word rows."""
    nrow = 64 // (32 // bits)
    out = np.empty((blocks.shape[0], nrow, 128), np.uint32)
    for r in range(nrow):
        for d in range(128):
            out[:, r, d] = blocks[:, 512 * (r // 4) + 256 * ((d // 4) % 2) + 64 * (r % 4) + 4 * (d // 8) + d % 4]
    return out.reshape(-1, 128)


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("k_axis,v_axis", [("channel", "token"), ("token", "channel")])
def test_layout_worked_example(orc, bits, k_axis, v_axis):
    L, D = 256, 128
    fmt = orc.make_format(bits, k_axis, v_axis, 128, D, 1, 4)
    x = _grid_data(L, D, bits)
    k = x[None, None]
    v = x[None, None]
    kc, vw, ksz, vsz = orc.quantize_pack(fmt, k, v, [L])
    code = ((np.arange(L)[:, None] * 3 + np.arange(D)[None, :]) % (1 << bits)).astype(np.uint32)
    # K: channel d of token t at bit bits*d of the token's row (little-endian bytes)
    per_byte = 8 // bits
    want_k = np.zeros((L, D * bits // 8), np.uint8)
    for j in range(per_byte):
        want_k |= (code[:, j::per_byte] << (bits * j)).astype(np.uint8)
    assert np.array_equal(_unblock_k(kc[0, 0], bits)[:L], want_k)
    # V: word w of channel d holds tokens w*tpw + j at bit bits*j
    tpw = 32 // bits
    want_v = np.zeros((L // tpw, D), np.uint32)
    for j in range(tpw):
        want_v |= code[j::tpw, :] << np.uint32(bits * j)
    assert np.array_equal(_unblock_v(vw[0, 0], bits)[:L // tpw], want_v)
    # every (s, z) is (1.0, 0.0)
    one = np.float16(1).view(np.uint16)
    assert np.all(ksz[..., 0] == one) and np.all(ksz[..., 1] == 0)
    assert np.all(vsz[..., 0] == one) and np.all(vsz[..., 1] == 0)


def test_layout_golden_bytes(orc):
    """Bytes written out by hand in tests/golden/layout_int4_int2.txt."""
    cases = _golden("layout_int4_int2.txt")
    for bits in (4, 2):
        codes = [int(c) for c in cases[f"int{bits}_codes"].split()]
        D = 128
        # token 0 carries the listed codes in channels 0..len-1, channel 127 = qmax, rest 0;
        # token-wise K groups so s = 1, z = 0
        qmax = (1 << bits) - 1
        row = np.zeros(D, np.float32)
        row[:len(codes)] = codes
        row[D - 1] = qmax
        x = np.tile(row, (128, 1))
        fmt = orc.make_format(bits, "token", "token", 128, D, 1, 4)
        kc, vw, _, _ = orc.quantize_pack(fmt, x[None, None], x[None, None], [128])
        # token 0's row starts the block (slot 0, first piece)
        want = bytes.fromhex(cases[f"int{bits}_k_row0_first_bytes"])
        assert bytes(kc[0, 0, 0, :len(want)]) == want
        # word-row 0, channel 1 is block word 1
        want_w = int(cases[f"int{bits}_v_word0_ch1"], 16)
        assert int(vw[0, 0, 0, 1]) == want_w


@pytest.mark.parametrize("bits", [4, 2])
def test_layout_block_positions_golden(orc, bits):
    """Hand-worked block positions of K row bytes and V words (golden file),
    on a cache whose token t, channel d code is (t + d) mod 2^b (token-wise
    groups, so s = 1, z = 0 and the stored codes are these values)."""
    cases = _golden("layout_int4_int2.txt")
    L, D, qm = 128, 128, (1 << bits) - 1
    t = np.arange(L)[:, None]
    d = np.arange(D)[None, :]
    code = (t + d) % (qm + 1)
    x = code.astype(np.float32)
    fmt = orc.make_format(bits, "token", "token", 128, D, 1, 4)
    kc, vw, _, _ = orc.quantize_pack(fmt, x[None, None], x[None, None], [L])
    per = 8 // bits
    tpw = 32 // bits
    for ent in cases[f"int{bits}_k_positions"].split(","):
        u, o, p = (int(z) for z in ent.split())
        want = sum(int(code[u, per * o + j]) << (bits * j) for j in range(per))
        assert int(kc[0, 0, 0, p]) == want, (bits, u, o, p)
    for ent in cases[f"int{bits}_v_positions"].split(","):
        r, ch, p = (int(z) for z in ent.split())
        want = sum(int(code[tpw * r + j, ch]) << (bits * j) for j in range(tpw))
        assert int(vw[0, 0, 0, p]) == want, (bits, r, ch, p)
    # the slot maps are permutations of the block's 64 slots, so the K block
    # order moves whole 16-byte pieces without overlap
    for b_, sl in _slot_tables().items():
        assert sorted(sl.tolist()) == list(range(64)), b_


# --------------------------------------------------------------------------
# attention: closed forms and torch's fp64 attention
# --------------------------------------------------------------------------

def _sdpa64(q, kh, vh, scale):
    qt = torch.from_numpy(q)[None, :, None, :]           # [1][R][1][D]
    kt = torch.from_numpy(kh)[None, None].expand(1, q.shape[0], -1, -1)
    vt = torch.from_numpy(vh)[None, None].expand(1, q.shape[0], -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    return o[0, :, 0, :].numpy()


@pytest.mark.parametrize("L", [1, 7, 300])
def test_attention_matches_torch_fp64(orc, L):
    rng = np.random.default_rng(L)
    q = rng.standard_normal((4, 128))
    kh = rng.standard_normal((L, 128)) * 2
    vh = rng.standard_normal((L, 128))
    got = orc.attention_f64(q, kh, vh, 1 / math.sqrt(128))
    want = _sdpa64(q, kh, vh, 1 / math.sqrt(128))
    assert np.allclose(got, want, rtol=1e-12, atol=1e-13)


def test_attention_closed_forms(orc):
    rng = np.random.default_rng(3)
    L, D = 500, 128
    kh = rng.standard_normal((L, D))
    vh = rng.standard_normal((L, D))
    # q = 0: uniform softmax, output = mean of V
    o = orc.attention_f64(np.zeros((2, D)), kh, vh, 0.1)
    m = np.array([math.fsum(vh[:, d]) / L for d in range(D)])
    assert np.allclose(o, m[None, :], rtol=0, atol=1e-14)
    # one-hot: score gap > 746 makes every other exp underflow to exactly 0
    q = np.full((1, D), 8.0)
    kk = np.full((L, D), -8.0)
    kk[123] = 8.0
    o = orc.attention_f64(q, kk, vh, 1.0)
    assert np.array_equal(o[0], vh[123])
    # L = 1: output is the single V row
    o = orc.attention_f64(rng.standard_normal((3, D)), kh[:1], vh[:1], 0.3)
    assert np.array_equal(o, np.repeat(vh[:1], 3, axis=0))
    # L = 0: zeros
    o = orc.attention_f64(rng.standard_normal((2, D)), kh[:0], vh[:0], 0.3)
    assert not o.any()


def _small_workload(bits, k_axis, v_axis, lens, seed=11, hkv=2, outliers=True):
    w = synth.Workload("t", len(lens), hkv, 4 * hkv, 128, list(lens), bits, k_axis, v_axis,
                       seed=seed, outliers=outliers)
    return w


@pytest.mark.parametrize("bits", [2, 4])
def test_decode_attention_vs_torch_and_gqa(orc, bits):
    w = _small_workload(bits, "channel", "token", [300, 0, 129])
    fmt = orc.fmt_of(w)
    k, v = w.kv_all("k"), w.kv_all("v")
    q = w.q_bf16()
    # make the 4 query heads of KV head 1 of batch 0 identical
    q[0, 4:8] = q[0, 4]
    cache = orc.quantize_pack(fmt, k, v, w.seq_lens)
    scale = 1 / math.sqrt(128)
    out = orc.decode_attention(fmt, q, cache, w.seq_lens, w.max_len, scale)
    qf = synth.bf16_bits_to_f32(q).astype(np.float64)
    for b, L in enumerate(w.seq_lens):
        for h in range(w.num_kv_heads):
            if L == 0:
                assert not out[b, 4 * h:4 * h + 4].any()
                continue
            kh = orc.dequantize_unit(fmt, "k", cache, b, h, L, w.max_len)
            vh = orc.dequantize_unit(fmt, "v", cache, b, h, L, w.max_len)
            want = _sdpa64(qf[b, 4 * h:4 * h + 4], kh, vh, scale)
            assert np.allclose(out[b, 4 * h:4 * h + 4], want, rtol=1e-11, atol=1e-13)
            # dequantised values are within half a quantisation step (plus the
            # cost of storing s, z in binary16) of the inputs
            s_max = cache[2][b, h, :(L + 127) // 128, :, 0].view(np.float16).astype(np.float64).max()
            assert np.abs(kh - k[b, h, :L]).max() <= 0.5 * s_max * 1.02 + 1e-2
    assert np.array_equal(out[0, 4], out[0, 5]) and np.array_equal(out[0, 4], out[0, 7])


def test_units_subset_matches_full(orc):
    w = _small_workload(4, "channel", "token", [256, 384])
    fmt = orc.fmt_of(w)
    cache = orc.quantize_pack(fmt, w.kv_all("k"), w.kv_all("v"), w.seq_lens)
    q = w.q_bf16()
    full = orc.decode_attention(fmt, q, cache, w.seq_lens, w.max_len, 0.088)
    part = orc.decode_attention(fmt, q, cache, w.seq_lens, w.max_len, 0.088, units=[(1, 1)])
    assert np.array_equal(part[1, 4:8], full[1, 4:8])
    assert not part[0].any()


# --------------------------------------------------------------------------
# the folds: exact in exact arithmetic (fp64 to 1e-12), and the group rule
# --------------------------------------------------------------------------

@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("k_axis", ["token", "channel"])
@pytest.mark.parametrize("v_axis", ["token", "channel"])
@pytest.mark.parametrize("group", [32, 64, 128])
def test_folded_equals_unfolded(orc, bits, k_axis, v_axis, group):
    w = _small_workload(bits, k_axis, v_axis, [300, 77], seed=group + bits)
    fmt = orc.fmt_of(w, group=group)
    cache = orc.quantize_pack(fmt, w.kv_all("k"), w.kv_all("v"), w.seq_lens)
    q = w.q_bf16()
    a = orc.decode_attention(fmt, q, cache, w.seq_lens, w.max_len, 1 / math.sqrt(128))
    f = orc.decode_attention_folded(fmt, q, cache, w.seq_lens, w.max_len, 1 / math.sqrt(128))
    rel = np.linalg.norm(a - f) / np.linalg.norm(a)
    assert rel < 1e-12


@pytest.mark.parametrize("k_axis,v_axis,group", [("channel", "channel", 128), ("token", "token", 32)])
def test_cross_group_accumulation_is_wrong(orc, k_axis, v_axis, group):
    """acc-fold partials accumulated across group boundaries give a different
    answer (rag-lover.com limits section), so the per-group rule matters."""
    w = _small_workload(2, k_axis, v_axis, [300], seed=5)
    fmt = orc.fmt_of(w, group=group)
    cache = orc.quantize_pack(fmt, w.kv_all("k"), w.kv_all("v"), w.seq_lens)
    q = w.q_bf16()
    a = orc.decode_attention(fmt, q, cache, w.seq_lens, w.max_len, 1 / math.sqrt(128))
    bad = orc.decode_attention_folded(fmt, q, cache, w.seq_lens, w.max_len, 1 / math.sqrt(128),
                                      bug=True)
    assert np.linalg.norm(a - bad) / np.linalg.norm(a) > 1e-3


# --------------------------------------------------------------------------
# paged layout: same codes, same answer as the contiguous one
# --------------------------------------------------------------------------

@pytest.mark.parametrize("bits", [2, 4])
def test_paged_equals_contiguous(orc, bits):
    lens = [200, 64, 1, 333]
    w = _small_workload(bits, "channel", "token", lens, seed=21)
    table, n_pages = synth.build_page_table(lens, 64, seed=9)
    k, v = w.kv_all("k"), w.kv_all("v")
    fc = orc.fmt_of(w)
    w.page_size = 64
    fp = orc.fmt_of(w)
    cc = orc.quantize_pack(fc, k, v, lens)
    cp = orc.quantize_pack(fp, k, v, lens, page_table=table, num_pages=n_pages)
    for b, L in enumerate(lens):
        for h in range(w.num_kv_heads):
            for which in "kv":
                a = orc.dequantize_unit(fc, which, cc, b, h, L, w.max_len)
                p = orc.dequantize_unit(fp, which, cp, b, h, L, w.max_len, page_table=table)
                assert np.array_equal(a, p)
    # byte placement: logical page p of sequence b lives in pool slot table[b][p]
    tpw = 32 // bits
    for b, L in enumerate(lens):
        for p in range((L + 63) // 64):
            ph = table[b, p]
            assert np.array_equal(cp[0][ph], cc[0][b, :, p])   # one 64-token code block
            assert np.array_equal(cp[1][ph], cc[1][b, :, p])
            assert np.array_equal(cp[3][ph], cc[3][b, :, 64 * p:64 * p + 64])
            if p % 2 == 0:  # channel-wise K pairs sit in a group's first page
                assert np.array_equal(cp[2][ph], cc[2][b, :, p // 2])
    q = w.q_bf16()
    oc = orc.decode_attention(fc, q, cc, lens, w.max_len, 0.088)
    op = orc.decode_attention(fp, q, cp, lens, w.max_len, 0.088, page_table=table)
    assert np.array_equal(oc, op)


@pytest.mark.parametrize("bits,group", [(2, 32), (4, 64)])
def test_paged_equals_contiguous_token_groups(orc, bits, group):
    """Token-wise K and V with 32- or 64-channel groups: a token's pairs move
    with its page, and the paged decode equals the contiguous one exactly."""
    lens = [200, 64, 1, 333]
    w = _small_workload(bits, "token", "token", lens, seed=23)
    table, n_pages = synth.build_page_table(lens, 64, seed=10)
    k, v = w.kv_all("k"), w.kv_all("v")
    fc = orc.fmt_of(w, group=group)
    w.page_size = 64
    fp = orc.fmt_of(w, group=group)
    cc = orc.quantize_pack(fc, k, v, lens)
    cp = orc.quantize_pack(fp, k, v, lens, page_table=table, num_pages=n_pages)
    for b, L in enumerate(lens):
        for p in range((L + 63) // 64):
            ph = table[b, p]
            for i in range(4):  # codes, words, and both tensors' pairs: one block each
                src = cc[i][b, :, p] if i < 2 else cc[i][b, :, 64 * p:64 * p + 64]
                assert np.array_equal(cp[i][ph], src), (b, p, i)
    q = w.q_bf16()
    oc = orc.decode_attention(fc, q, cc, lens, w.max_len, 0.088)
    op = orc.decode_attention(fp, q, cp, lens, w.max_len, 0.088, page_table=table)
    assert np.array_equal(oc, op)
    assert np.abs(oc).max() > 0


def test_bf16_attention_vs_torch(orc):
    rng = np.random.default_rng(5)
    B, H, L, D = 2, 2, 150, 128
    q = synth.f32_to_bf16_bits(rng.standard_normal((B, 4 * H, D)).astype(np.float32))
    k = synth.f32_to_bf16_bits(rng.standard_normal((B, H, L, D)).astype(np.float32))
    v = synth.f32_to_bf16_bits(rng.standard_normal((B, H, L, D)).astype(np.float32))
    lens = [150, 40]
    out = orc.decode_attention_bf16(q, k, v, lens, L, 0.088, H)
    for b in range(B):
        for h in range(H):
            want = _sdpa64(synth.bf16_bits_to_f32(q[b, 4 * h:4 * h + 4]).astype(np.float64),
                           synth.bf16_bits_to_f32(k[b, h, :lens[b]]).astype(np.float64),
                           synth.bf16_bits_to_f32(v[b, h, :lens[b]]).astype(np.float64), 0.088)
            assert np.allclose(out[b, 4 * h:4 * h + 4], want, rtol=1e-11, atol=1e-13)


def test_window_attention_vs_torch_and_special_cases(orc):
    """The residual-window decode: whole groups dequantised from the cache, the
    rest from the bf16 window. Pinned to torch's fp64 attention on the
    concatenation, to the cache-only decode when the window is empty, and to
    the bf16 decode when no group is complete."""
    rng = np.random.default_rng(11)
    B, H, D = 3, 2, 128
    lens = [300, 256, 77]  # window 44, empty, everything in the window
    Lmax = 300
    w = _small_workload(2, "channel", "token", [Lmax] * B)
    fmt = orc.fmt_of(w)
    k, v = w.kv_all("k"), w.kv_all("v")
    lq = [L - L % 128 for L in lens]
    cache = orc.quantize_pack(fmt, k, v, lq)
    kw = synth.f32_to_bf16_bits(rng.standard_normal((B, H, 128, D)).astype(np.float32))
    vw = synth.f32_to_bf16_bits(rng.standard_normal((B, H, 128, D)).astype(np.float32))
    q = synth.f32_to_bf16_bits(rng.standard_normal((B, 4 * H, D)).astype(np.float32))
    scale = 1 / math.sqrt(128)
    out = orc.decode_attention_window(fmt, q, cache, kw, vw, lens, Lmax, scale)
    qf = synth.bf16_bits_to_f32(q).astype(np.float64)
    for b, L in enumerate(lens):
        r = L - lq[b]
        for h in range(H):
            kh = np.concatenate([orc.dequantize_unit(fmt, "k", cache, b, h, lq[b], Lmax),
                                 synth.bf16_bits_to_f32(kw[b, h, :r]).astype(np.float64)])
            vh = np.concatenate([orc.dequantize_unit(fmt, "v", cache, b, h, lq[b], Lmax),
                                 synth.bf16_bits_to_f32(vw[b, h, :r]).astype(np.float64)])
            want = _sdpa64(qf[b, 4 * h:4 * h + 4], kh, vh, scale)
            assert np.allclose(out[b, 4 * h:4 * h + 4], want, rtol=1e-11, atol=1e-13)
    # empty window: the cache-only decode
    full = orc.decode_attention(fmt, q, cache, lq, Lmax, scale)
    assert np.allclose(out[1], full[1], rtol=1e-12, atol=1e-14)
    # no complete group: the bf16 decode of the window alone
    bfo = orc.decode_attention_bf16(q, kw, vw, [0, 0, 77], 128, scale, H)
    assert np.allclose(out[2], bfo[2], rtol=1e-12, atol=1e-14)
