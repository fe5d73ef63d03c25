"""The C ABI without a GPU: the library loads, exports every function that
include/kvq.h declares, and rejects bad arguments synchronously, before any
HIP call (so these checks run on a host with no device)."""
import ctypes
import os
import re

import pytest

import bit_quantized_kv_int2_amd as kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, NULLP, BADFMT, BADSHAPE, MISALIGNED, WORKSPACE = 0, 1, 2, 3, 4, 5


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(kvq.LIB_PATH):
        from bit_quantized_kv_int2_amd import build
        build.build()
    return kvq.lib()


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "kvq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_exports_every_declared_function(L):
    names = _declared_functions()
    assert {"kv_quantize_pack", "decode_attention_quant", "decode_attention_bf16"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_stream_read_validation_without_gpu(L):
    f = L.kvq_stream_read
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    A = 4096
    assert f(None, 16, A, None) == NULLP
    assert f(A, 16, None, None) == NULLP
    assert f(A + 8, 16, A, None) == MISALIGNED
    assert f(A, 16, A + 2, None) == MISALIGNED
    assert f(A, 24, A, None) == BADSHAPE
    assert f(A, 0, A, None) == OK  # nothing to read, nothing launched


def test_issue_probe_validation_without_gpu(L):
    f = L.kvq_issue_probe
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    A = 4096
    assert f(0, 10, 4, None, None) == NULLP
    assert f(0, 10, 4, A + 2, None) == MISALIGNED
    for mode, iters, blocks in [(-1, 10, 4), (4, 10, 4), (0, 0, 4), (1, 10, 0), (2, 10, 65536)]:
        assert f(mode, iters, blocks, A, None) == BADSHAPE, (mode, iters, blocks)


def test_layout_version_and_status_strings(L):
    assert L.kvq_layout_version() == kvq.LAYOUT_VERSION
    for s in range(7):
        assert L.kvq_status_string(s)


def test_format_checks(L):
    good = kvq.make_format(2, "channel", "token", 8)
    assert kvq.kvq_check_format(good) == OK
    for field, bad in [("bits", 3), ("bits", 8), ("group", 64), ("head_dim", 64),
                       ("num_q_heads", 16), ("page_size", 32), ("layout_version", 1),
                       ("layout_version", 3),
                       ("k_axis", 2), ("num_kv_heads", 0)]:
        f = kvq.make_format(2, "channel", "token", 8)
        setattr(f, field, bad)
        assert kvq.kvq_check_format(f) == BADFMT, field
    assert L.kvq_check_format(None) == NULLP


def test_cache_sizes(L):
    f = kvq.make_format(4, "channel", "token", 8)
    kc, vc, ks, vs = kvq.kvq_cache_sizes(f, 128, 32768)
    assert kc == vc == 128 * 8 * 32768 * 64
    assert ks == 128 * 8 * 256 * 128 * 4 and vs == 128 * 8 * 32768 * 4
    f2 = kvq.make_format(2, "token", "channel", 8)
    kc, vc, ks, vs = kvq.kvq_cache_sizes(f2, 3, 1000)   # padded to 1024 tokens
    assert kc == 3 * 8 * 1024 * 32 and ks == 3 * 8 * 1024 * 4 and vs == 3 * 8 * 8 * 128 * 4
    fp = kvq.make_format(4, "channel", "token", 8, page_size=64)
    kc, vc, ks, vs = kvq.kvq_cache_sizes(fp, 0, 0, 100)
    assert kc == 100 * 8 * 64 * 64 and ks == 100 * 8 * 128 * 4 and vs == 100 * 8 * 64 * 4


def test_small_token_wise_groups(L):
    # 32 or 64 channels per group only when K and V are both token-wise
    # (contiguous or paged: a token's pairs sit in its page)
    for gsz in (32, 64):
        assert kvq.kvq_check_format(kvq.make_format(2, "token", "token", 2, group=gsz)) == OK
        assert kvq.kvq_check_format(kvq.make_format(4, "channel", "token", 2, group=gsz)) == BADFMT
        assert kvq.kvq_check_format(kvq.make_format(4, "token", "channel", 2, group=gsz)) == BADFMT
        fp = kvq.make_format(2, "token", "token", 2, group=gsz, page_size=64)
        assert kvq.kvq_check_format(fp) == OK
        assert kvq.kvq_check_format(kvq.make_format(2, "token", "channel", 2, group=gsz,
                                                    page_size=64)) == BADFMT
        kc, vc, ks, vs = kvq.kvq_cache_sizes(kvq.make_format(4, "token", "token", 2, group=gsz), 3, 1000)
        assert kc == vc == 3 * 2 * 1024 * 64
        assert ks == vs == 3 * 2 * 1024 * (128 // gsz) * 4
        kc, vc, ks, vs = kvq.kvq_cache_sizes(fp, 0, 0, 7)  # 7 pages of 64 tokens x 2 heads
        assert kc == vc == 7 * 2 * 64 * 32
        assert ks == vs == 7 * 2 * 64 * (128 // gsz) * 4
    for bad in (16, 96, 256):
        assert kvq.kvq_check_format(kvq.make_format(2, "token", "token", 2, group=bad)) == BADFMT


def _auto_ws(rows, ns_auto, slots):
    items = max(-(-rows // 8) * 8 * ns_auto, 2 * slots + rows)
    return 16 + -(-rows * 4 // 16) * 16 + items * 4 * 130 * 4


def test_split_plan_and_workspace(L):
    f = kvq.make_format(2, "channel", "token", 8)
    ns = kvq.kvq_plan_splits(f, 128, 32768)
    assert 1 <= ns <= 128
    # one split per row: no merge, no workspace (the rows fill the chip)
    assert ns == 1 and kvq.kvq_workspace_size(f, 128, 32768) == 0
    # a split plan runs on the device: a 16-byte header, one int32 per
    # (sequence, KV head) row, and partials (4 x 130 floats) for each of the
    # grid's max(rows * ns, 2 slots + rows) work-items
    assert kvq.kvq_workspace_size(f, 16, 4096) == _auto_ws(16 * 8, 8, 1024)
    # a single sequence is split finely enough to occupy the chip
    assert kvq.kvq_plan_splits(kvq.make_format(4, num_kv_heads=1), 1, 32768) >= 64
    assert kvq.kvq_plan_splits(kvq.make_format(4, num_kv_heads=1), 1, 1024) == 4
    # the auto plan gives one round of resident work-groups (256 CUs x 4 for INT2,
    # x 3 for INT4): no split at 1024 units, 8 / 6 splits at 128
    assert kvq.kvq_plan_splits(f, 128, 32768) == 1
    assert kvq.kvq_plan_splits(kvq.make_format(4, "channel", "token", 8), 128, 32768) == 1
    share2, share4 = kvq.make_format(2, num_kv_heads=1), kvq.make_format(4, num_kv_heads=1)
    assert kvq.kvq_plan_splits(share2, 128, 32768) == 8
    assert kvq.kvq_plan_splits(share4, 128, 32768) == 6
    assert kvq.kvq_plan_splits(kvq.make_format(2, "channel", "channel", 1), 128, 32768) == 8
    assert kvq.kvq_plan_splits(kvq.make_format(4, "channel", "channel", 1), 128, 32768) == 6
    # the workspace also covers the bf16 decode's plan (1024 work-groups: 8
    # splits), and with explicit counts it is the (row, split) partials alone
    assert kvq.kvq_workspace_size(share4, 128, 32768) == max(_auto_ws(128, 6, 768),
                                                            128 * 4 * 8 * 130 * 4)
    assert kvq.kvq_workspace_size(share4, 128, 32768, 6) == 128 * 4 * 6 * 130 * 4
    # explicit splits: any count from 1 to ceil(L / 256); one split needs no workspace
    assert kvq.kvq_workspace_size(f, 2, 32768, 1) == 0
    assert kvq.kvq_workspace_size(f, 2, 32768, 3) == 2 * 32 * 3 * 130 * 4
    with pytest.raises(kvq.KvqError):
        kvq.kvq_workspace_size(f, 2, 1024, 5)
    # a decode launch is a 1-D grid of fewer than 2^24 work-groups of 256
    # work-items (a 32-bit count): splits x rows, rows (sequences x KV heads)
    # padded to a multiple of 8
    assert kvq.kvq_workspace_size(f, 4096, 1 << 20, 256) == 4096 * 32 * 256 * 130 * 4
    with pytest.raises(kvq.KvqError):
        kvq.kvq_workspace_size(f, 4096, 1 << 20, 512)
    with pytest.raises(kvq.KvqError):
        kvq.kvq_workspace_size(f, 2, 1024, -1)


def test_auto_plan_rule(L):
    """The quantised decode's auto plan (made on the device; kvq_auto_plan is
    its host copy): the max_len plan's split for about equal lengths, whole
    2048-token chunks of about H sum(L) / (2 slots) tokens for a ragged batch,
    and never more work-items than the grid the call launches."""
    import numpy as np
    import synth
    for bits in (2, 4):
        slots = 256 * (4 if bits == 2 else 3)
        f = kvq.make_format(bits, "channel", "token", 8)
        # 1024 rows fill the chip: one split per row whatever the lengths
        assert kvq.kvq_auto_plan(f, [32768] * 128, 32768) == (32768, 1024, 1024)
        assert kvq.kvq_auto_plan(f, [32768] + [100] * 127, 32768) == (32768, 1024, 1024)
        # 16 x 8 rows: the max_len plan splits them, so the plan is made on the
        # device; equal lengths and a mild spread keep the max_len split
        S, items, grid = kvq.kvq_auto_plan(f, [4096] * 16, 4096)
        ns = kvq.kvq_plan_splits(f, 16, 4096)
        assert ns == -(-slots // 128) and S == -(-16 // ns) * 256
        assert items == 128 * -(-4096 // S) and grid == max(128 * ns, 2 * slots + 128)
        assert kvq.kvq_auto_plan(f, list(range(3000, 3000 + 16 * 20, 20)), 3320)[0] == \
            -(-(-(-3320 // 256)) // kvq.kvq_plan_splits(f, 16, 3320)) * 256
        # the long-context paged batch: 64 sequences log-uniform in [1K, 128K]
        fp = kvq.make_format(bits, "channel", "token", 8, page_size=64)
        lens = synth.paged_long(0).seq_lens
        Lmax = max(lens)
        S, items, grid = kvq.kvq_auto_plan(fp, lens, Lmax)
        t = -(-8 * sum(lens) // (2 * slots))
        assert S == 2048 * max(1, -(-t // 2048))
        assert items == sum(8 * -(-L // S) for L in lens) <= grid
        ns = kvq.kvq_plan_splits(fp, 64, Lmax)
        assert ns >= 2 and grid == max(64 * 8 * ns, 2 * slots + 64 * 8)
        # one long sequence among short ones, empty and clamped lengths
        assert kvq.kvq_auto_plan(f, [131072] + [1024] * 63, 131072)[0] == 2048
        assert kvq.kvq_auto_plan(f, [0] * 8, 4096)[1] == 0
        assert kvq.kvq_auto_plan(f, [-5, 99999999] + [32768] * 126, 32768) == \
            kvq.kvq_auto_plan(f, [0, 32768] + [32768] * 126, 32768)
        # many random batches: the items always fit the grid; the split is the
        # auto split or whole chunks below it
        rng = np.random.default_rng(bits)
        for trial in range(300):
            B = int(rng.integers(1, 300))
            H = int(rng.choice([1, 2, 8]))
            Lmax = int(rng.integers(1, 300000))
            ff = kvq.make_format(bits, "channel", "token", H)
            kind = trial % 3
            if kind == 0:
                lens = rng.integers(0, Lmax + 1, B)
            elif kind == 1:
                lens = np.exp(rng.uniform(0, np.log(Lmax + 1), B)).astype(np.int64)
            else:
                lens = np.where(rng.random(B) < 0.1, Lmax, rng.integers(0, max(1, Lmax // 50), B))
            lens = np.minimum(lens, Lmax)
            S, items, grid = kvq.kvq_auto_plan(ff, lens, Lmax)
            ns = kvq.kvq_plan_splits(ff, B, Lmax)
            auto_S = -(-(-(-Lmax // 256)) // ns) * 256
            assert items <= grid, (B, H, Lmax, S, items, grid)
            assert items == sum(H * -(-int(L) // S) for L in lens if L > 0)
            if ns == 1:
                assert S == auto_S and grid == -(-B * H // 8) * 8
            else:
                assert S == auto_S or (S % 2048 == 0 and S < auto_S)
                assert grid == max(-(-B * H // 8) * 8 * ns, 2 * slots + B * H)
    z = ctypes.c_int32()
    f = kvq.make_format(2, "channel", "token", 8)
    assert L.kvq_auto_plan(ctypes.byref(f), 4, 1024, None, ctypes.byref(z), ctypes.byref(z),
                           ctypes.byref(z)) == NULLP
    assert L.kvq_auto_plan(ctypes.byref(f), 0, 1024, None, ctypes.byref(z), ctypes.byref(z),
                           ctypes.byref(z)) == OK


def test_split_plan_for_known_lengths(L):
    """Host-side plan over known lengths: the auto plan for (near-)equal lengths,
    splits of whole 2048-token chunks sized to half the mean work per slot for a
    ragged batch, and always a count the decode accepts."""
    import synth
    for bits in (2, 4):
        f = kvq.make_format(bits, "channel", "token", 8)
        auto = kvq.kvq_plan_splits(f, 128, 32768)
        assert kvq.kvq_plan_splits_for_lengths(f, [32768] * 128, 32768) == auto
        mild = list(range(30000, 30000 + 128 * 20, 20))
        assert kvq.kvq_plan_splits_for_lengths(f, mild, 32768) == auto
        share = kvq.make_format(bits, num_kv_heads=1)
        assert kvq.kvq_plan_splits_for_lengths(share, [32768] * 128, 32768) == \
            kvq.kvq_plan_splits(share, 128, 32768)
        # the long-context paged batch: 64 sequences, log-uniform in [1K, 128K]
        fp = kvq.make_format(bits, "channel", "token", 8, page_size=64)
        lens = synth.paged_long(0).seq_lens
        Lmax = max(lens)
        ns = kvq.kvq_plan_splits_for_lengths(fp, lens, Lmax)
        slots = 256 * (4 if bits == 2 else 3)
        target = 8 * sum(lens) / (2 * slots)
        k0 = max(1, int(target / 2048 + 0.5))
        quanta = -(-Lmax // 256)                  # 256-token units of max_len

        def count(chunks):                        # splits the decode makes of that length
            req = -(-quanta // (8 * chunks))
            return -(-Lmax // (256 * -(-quanta // req)))
        cands = [count(k) for k in (k0, k0 + 1, k0 - 1) if k >= 1]
        want = next((c for c in cands if c % 2), next((c for c in cands if c % 4 == 2), cands[0]))
        assert ns == want
        assert ns % 2 == 1 or ns % 4 == 2
        assert ns > kvq.kvq_plan_splits(fp, 64, Lmax)
        kvq.kvq_workspace_size(fp, 64, Lmax, ns)  # accepted as an explicit count
        # one long sequence among short ones: one- or two-chunk splits
        assert kvq.kvq_plan_splits_for_lengths(f, [131072] + [1024] * 63, 131072) in (32, 64)
        # lengths are clamped to [0, max_len]; empty batches and all-empty lengths
        assert kvq.kvq_plan_splits_for_lengths(f, [-5, 99999999] + [32768] * 126, 32768) == \
            kvq.kvq_plan_splits_for_lengths(f, [0, 32768] + [32768] * 126, 32768)
        assert kvq.kvq_plan_splits_for_lengths(f, [], 32768) == kvq.kvq_plan_splits(f, 0, 32768)
        assert kvq.kvq_plan_splits_for_lengths(f, [0] * 8, 4096) == kvq.kvq_plan_splits(f, 8, 4096)
    n = ctypes.c_int32()
    f = kvq.make_format(2, "channel", "token", 8)
    assert L.kvq_plan_splits_for_lengths(ctypes.byref(f), 4, 1024, None, ctypes.byref(n)) == NULLP
    assert L.kvq_plan_splits_for_lengths(ctypes.byref(f), 0, 1024, None, ctypes.byref(n)) == OK
    arr = (ctypes.c_int32 * 2)(5, 6)
    assert L.kvq_plan_splits_for_lengths(ctypes.byref(f), 2, 1024, arr, None) == NULLP
    assert L.kvq_plan_splits_for_lengths(ctypes.byref(f), -1, 1024, arr, ctypes.byref(n)) == BADSHAPE


def _call_decode(L, fmt, q=16, cache=(16, 16, 16, 16), lens=16, table=None, maxp=0, B=1,
                 max_len=128, out=16, od=0, ns=0, ws=None, wsb=0):
    c = kvq.Cache(*cache) if cache is not None else None
    return L.decode_attention_quant(ctypes.byref(fmt) if fmt is not None else None, q,
                                    ctypes.byref(c) if c is not None else None, lens, table, maxp,
                                    B, max_len, ctypes.c_float(0.088), out, od, ns, ws, wsb, None)


def test_decode_validation_without_gpu(L):
    f = kvq.make_format(4, "channel", "token", 1)
    A = 4096  # fake, 16-byte aligned addresses: never dereferenced on failure paths
    assert _call_decode(L, None) == NULLP
    assert _call_decode(L, f, q=None) == NULLP
    assert _call_decode(L, f, cache=(A, A, None, A)) == NULLP
    assert _call_decode(L, f, cache=(A, A + 4, A, A)) == MISALIGNED
    assert _call_decode(L, f, q=A + 2, cache=(A, A, A, A), lens=A, out=A) == MISALIGNED
    assert _call_decode(L, f, cache=(A, A, A, A), lens=None, out=A, q=A) == NULLP
    assert _call_decode(L, f, cache=(A, A, A, A), lens=A, out=A, q=A, od=7) == BADFMT
    assert _call_decode(L, f, cache=(A, A, A, A), lens=A, out=A, q=A, B=-1) == BADSHAPE
    # needs a workspace: 2 splits requested, none given
    assert _call_decode(L, f, cache=(A, A, A, A), lens=A, out=A, q=A, max_len=4096,
                        ns=2) == WORKSPACE
    assert _call_decode(L, f, cache=(A, A, A, A), lens=A, out=A, q=A, max_len=4096, ns=2,
                        ws=A, wsb=10) == WORKSPACE
    # paged formats need a page table that covers max_len
    fp = kvq.make_format(4, "channel", "token", 1, page_size=64)
    assert _call_decode(L, fp, cache=(A, A, A, A), lens=A, out=A, q=A) == NULLP
    assert _call_decode(L, fp, cache=(A, A, A, A), lens=A, out=A, q=A, table=A, maxp=1,
                        max_len=4096) == BADSHAPE
    bad = kvq.make_format(3, "channel", "token", 1)
    assert _call_decode(L, bad, cache=(A, A, A, A), lens=A, out=A, q=A) == BADFMT


def test_grid_limits_without_gpu(L):
    """Grids must count their work-items in 32 bits, checked before any launch:
    2^24 decode work-groups of 256 work-items is one grid too many, and the
    merge of the window path (always launched) needs batch * Hq * 128 < 2^32."""
    A = 4096
    c = kvq.Cache(A, A, A, A)
    n = ctypes.c_size_t()
    f = kvq.make_format(2, "channel", "token", 64)
    # 32768 sequences x 64 KV heads x 8 splits of 256 tokens = 2^24 work-groups
    assert L.kvq_workspace_size(ctypes.byref(f), 32768, 2048, 8, ctypes.byref(n)) == BADSHAPE
    assert L.kvq_workspace_size(ctypes.byref(f), 32768, 2048, 7, ctypes.byref(n)) == OK
    assert L.decode_attention_quant(ctypes.byref(f), A, ctypes.byref(c), A, None, 0, 32768, 2048,
                                    ctypes.c_float(0.1), A, 0, 8, A, 1 << 40, None) == BADSHAPE
    # one split: 65535 x 129 KV heads is 8.45 M decode work-groups (fits), but
    # the window path's merge would run 65535 x 516 rows of 128 work-items
    fw = kvq.make_format(2, "channel", "token", 129)
    assert L.decode_attention_quant_window(ctypes.byref(fw), A, ctypes.byref(c), A, A, A, None, 0,
                                           65535, 128, ctypes.c_float(0.1), A, 0, 1, A, 1 << 40,
                                           None) == BADSHAPE


def test_noalloc_limit_without_gpu(L):
    """decode_attention_quant_noalloc rejects calls whose split partials do
    not fit its scratch array before any HIP call, and does nothing for an
    empty batch (both paths run here, where there is no device)."""
    f = kvq.make_format(4, "channel", "token", 8)
    A = 4096
    c = kvq.Cache(A, A, A, A)
    limit = 32 << 20

    def call(B, max_len, ns):
        return L.decode_attention_quant_noalloc(ctypes.byref(f), A, ctypes.byref(c), A, None, 0,
                                                B, max_len, ctypes.c_float(0.1), A, 0, ns, None)
    # 127 sequences x 32 query heads x 16 splits x 130 floats: just over the limit
    assert kvq.kvq_workspace_size(f, 127, 4096, 16) > limit
    assert call(127, 4096, 16) == WORKSPACE
    # 126 sequences fit (the check is on the bytes, not the shape)
    assert kvq.kvq_workspace_size(f, 126, 4096, 16) <= limit
    assert call(0, 4096, 16) == OK
    assert call(-1, 4096, 16) == BADSHAPE
    assert L.decode_attention_quant_noalloc(None, A, ctypes.byref(c), A, None, 0, 1, 128,
                                            ctypes.c_float(0.1), A, 0, 0, None) == NULLP


def test_pack_and_bf16_validation_without_gpu(L):
    f = kvq.make_format(2, "token", "channel", 2)
    A = 4096
    c = kvq.Cache(A, A, A, A)
    assert L.kv_quantize_pack(ctypes.byref(f), None, A, A, None, 0, 1, 128, ctypes.byref(c),
                              None) == NULLP
    assert L.kv_quantize_pack(ctypes.byref(f), A + 8, A, A, None, 0, 1, 128, ctypes.byref(c),
                              None) == MISALIGNED
    assert L.kv_quantize_pack(ctypes.byref(f), A, A, A, None, 0, 1, 128, None, None) == NULLP
    assert L.kv_quantize_pack(ctypes.byref(f), A, A, A, None, 0, 1, -5, ctypes.byref(c),
                              None) == BADSHAPE
    # nothing to do: no launch, OK
    assert L.kv_quantize_pack(ctypes.byref(f), A, A, A, None, 0, 0, 128, ctypes.byref(c),
                              None) == OK
    assert L.decode_attention_bf16(ctypes.byref(f), A, None, A, A, None, 0, 1, 128,
                                   ctypes.c_float(0.1), A, 0, 0, None, 0, None) == NULLP
    assert L.decode_attention_bf16(ctypes.byref(f), A, A, A, A, None, 0, 1, 128,
                                   ctypes.c_float(float("nan")), A, 0, 0, None, 0, None) == BADSHAPE


HIP_ERR = 6


@pytest.mark.skipif(os.path.exists("/dev/kfd"),
                    reason="host-only: its fake device addresses must never meet a device")
def test_injected_hip_failure_without_gpu(L):
    """The KVQ_ERR_HIP path of every entry point that launches: with an error
    code injected, each passes its host checks, then reports that code
    instead of its first HIP call; argument errors still come first."""
    A = 4096
    c = kvq.Cache(A, A, A, A)
    code = 719  # hipErrorLaunchFailure
    f = kvq.make_format(2, "channel", "token", 8)
    fp = kvq.make_format(2, "token", "token", 8, page_size=64)
    big = 1 << 40
    sf = ctypes.c_float(0.088)
    calls = {
        "pack": lambda: L.kv_quantize_pack(ctypes.byref(f), A, A, A, None, 0, 2, 300,
                                           ctypes.byref(c), None),
        "pack_paged": lambda: L.kv_quantize_pack(ctypes.byref(fp), A, A, A, A, 8, 2, 300,
                                                 ctypes.byref(c), None),
        "decode_one_split": lambda: _call_decode(L, f, cache=(A,) * 4, lens=A, out=A, q=A,
                                                 max_len=4096, ns=1),
        "decode_splits": lambda: _call_decode(L, f, cache=(A,) * 4, lens=A, out=A, q=A,
                                              max_len=4096, ns=4, ws=A, wsb=big),
        "decode_auto": lambda: _call_decode(L, f, cache=(A,) * 4, lens=A, out=A, q=A,
                                            max_len=32768, ns=0, ws=A, wsb=big),
        "decode_fp8": lambda: L.decode_attention_quant_fp8(ctypes.byref(f), A, ctypes.byref(c), A,
                                                           None, 0, 2, 4096, sf, A, 1, 2, A, big,
                                                           None),
        "noalloc_splits": lambda: L.decode_attention_quant_noalloc(
            ctypes.byref(f), A, ctypes.byref(c), A, None, 0, 2, 4096, sf, A, 0, 4, None),
        "noalloc_one_split": lambda: L.decode_attention_quant_noalloc(
            ctypes.byref(f), A, ctypes.byref(c), A, None, 0, 2, 4096, sf, A, 0, 1, None),
        "bf16": lambda: L.decode_attention_bf16(ctypes.byref(f), A, A, A, A, None, 0, 2, 4096, sf,
                                                A, 0, 2, A, big, None),
        "append": lambda: L.kv_append(ctypes.byref(f), A, A, A, None, 0, 2, 4096,
                                      ctypes.byref(c), A, A, None),
        "window": lambda: L.decode_attention_quant_window(ctypes.byref(f), A, ctypes.byref(c), A,
                                                          A, A, None, 0, 2, 4096, sf, A, 0, 2, A,
                                                          big, None),
        "stream_read": lambda: L.kvq_stream_read(A, 1 << 20, A, None),
        "issue_probe": lambda: L.kvq_issue_probe(0, 10, 4, A, None),
    }
    try:
        for i, (name, call) in enumerate(calls.items()):
            kvq.kvq_debug_inject_hip_error(code + i)  # a new code per call: none is stale
            assert call() == HIP_ERR, name
            assert L.kvq_last_hip_error() == code + i, name
        kvq.kvq_debug_inject_hip_error(code)
        # argument errors are reported before the HIP step
        assert _call_decode(L, f, q=None) == NULLP
        assert L.kvq_stream_read(A, 24, A, None) == BADSHAPE
        # calls with nothing to launch succeed without reaching it
        assert L.kvq_stream_read(A, 0, A, None) == OK
        assert _call_decode(L, f, cache=(A,) * 4, lens=A, out=A, q=A, B=0, ns=1) == OK
        assert L.kv_quantize_pack(ctypes.byref(f), A, A, A, None, 0, 0, 128, ctypes.byref(c),
                                  None) == OK
        # the binding names the injected code
        assert calls["stream_read"]() == HIP_ERR
        msg = str(kvq.KvqError(HIP_ERR, "kvq_stream_read"))
        assert "KVQ_ERR_HIP" in msg and str(code) in msg
        assert L.kvq_status_string(HIP_ERR) == b"HIP launch failed"
    finally:
        kvq.kvq_debug_inject_hip_error(0)


def test_calls_without_library_fail_loudly(monkeypatch, tmp_path):
    """The binding has no fallback: with the library missing, calls raise."""
    import importlib
    monkeypatch.setattr(kvq, "_lib", None)
    monkeypatch.setattr(kvq, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError):
        kvq.lib()


def test_product_path_does_not_reach_the_oracle(L):
    """Nothing in the package (binding, build script, HIP sources) imports,
    loads or links the CPU oracle, and the built library needs no oracle
    symbol: the oracle is test infrastructure only."""
    pkg = os.path.join(ROOT, "bit_quantized_kv_int2_amd")
    pat = re.compile(r"\boracle\b|liboracle|\borc_")
    for dirpath, _, files in os.walk(pkg):
        for name in files:
            if name.endswith((".py", ".hip", ".h", ".cpp", ".c")):
                text = open(os.path.join(dirpath, name)).read()
                assert not pat.search(text), os.path.join(dirpath, name)
    with open(kvq.LIB_PATH, "rb") as f:
        blob = f.read()
    assert b"liboracle" not in blob and b"orc_attention" not in blob
