"""Seeded synthetic inputs for INT2/INT4 decode attention.

This module is shared by the CPU oracle and the GPU library's tests and
benchmark. It only draws random numbers in the shapes the workloads need; it
holds none of the quantisation or attention arithmetic.

Every array is addressable by slice: the values of one (stream, b, h) slice
come from their own numpy ``SeedSequence([seed, stream, b, h])`` and do not
depend on which other slices are drawn, so a test can regenerate a single
(batch row, KV head) of a huge workload without drawing the rest.

Streams: 0 query, 1 K, 2 V, 3 K outlier mask, 4 K outlier offset,
5 sequence lengths, 6 page permutation. Layer ``l`` of a multi-layer workload
adds ``16 * l`` to the K/V/outlier streams.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

S_Q, S_K, S_V, S_OMASK, S_OOFF, S_LENS, S_PERM = 0, 1, 2, 3, 4, 5, 6


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def normal_f32(shape, *key: int) -> np.ndarray:
    """Standard normal float32 draws for one slice."""
    return _rng(*key).standard_normal(shape, dtype=np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bit patterns.

    Used only to turn drawn float32 queries into the bf16 inputs the workloads
    specify (both sides then read the same bits). NaN is not expected here.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Workload:
    """Shape and distribution of one synthetic decode-attention workload."""

    name: str
    batch: int
    num_kv_heads: int
    num_q_heads: int
    head_dim: int
    seq_lens: list
    bits: int
    k_axis: str = "channel"   # "channel" or "token"
    v_axis: str = "token"
    seed: int = 0
    outliers: bool = False     # 2% of K channels get a per-channel offset ~ N(0, 2^2)
    outlier_frac: float = 0.02
    outlier_sigma: float = 2.0
    layer: int = 0
    page_size: int = 0         # 0: contiguous cache; 64: paged
    extra: dict = field(default_factory=dict)

    @property
    def max_len(self) -> int:
        return int(max(self.seq_lens)) if len(self.seq_lens) else 0

    @property
    def group_ratio(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def stream(self, s: int) -> int:
        return s + 16 * self.layer if s in (S_K, S_V, S_OMASK, S_OOFF) else s

    # ---- queries -------------------------------------------------------
    def q_f32(self, b: int) -> np.ndarray:
        """[Hq][D] float32 query of batch row b (before bf16 rounding)."""
        return normal_f32((self.num_q_heads, self.head_dim), self.seed, S_Q, b)

    def q_bf16(self) -> np.ndarray:
        """[B][Hq][D] bf16 bit patterns (uint16)."""
        out = np.empty((self.batch, self.num_q_heads, self.head_dim), np.uint16)
        for b in range(self.batch):
            out[b] = f32_to_bf16_bits(self.q_f32(b))
        return out

    # ---- K/V -----------------------------------------------------------
    def outlier_offsets(self) -> np.ndarray:
        """[Hkv][D] float32 per-channel K offsets (0 where a channel is not an outlier)."""
        if not self.outliers:
            return np.zeros((self.num_kv_heads, self.head_dim), np.float32)
        u = _rng(self.seed, self.stream(S_OMASK)).random((self.num_kv_heads, self.head_dim))
        off = normal_f32((self.num_kv_heads, self.head_dim), self.seed, self.stream(S_OOFF))
        off = (off.astype(np.float64) * self.outlier_sigma).astype(np.float32)
        return np.where(u < self.outlier_frac, off, np.float32(0)).astype(np.float32)

    def kv_unit(self, which: str, b: int, h: int, length: int | None = None,
                offsets: np.ndarray | None = None) -> np.ndarray:
        """[L][D] float32 K or V values of one (batch row, KV head).

        ``length`` defaults to max_len; rows past a sequence's length are
        drawn all the same (they are never read)."""
        L = self.max_len if length is None else length
        s = S_K if which == "k" else S_V
        x = normal_f32((L, self.head_dim), self.seed, self.stream(s), b, h)
        if which == "k" and self.outliers:
            off = self.outlier_offsets() if offsets is None else offsets
            x += off[h][None, :]
        return x

    def kv_row(self, which: str, b: int, length: int | None = None,
               offsets: np.ndarray | None = None, threads: int | None = None,
               out: np.ndarray | None = None) -> np.ndarray:
        """[Hkv][L][D] float32 K or V of batch row b (threaded over KV heads)."""
        L = self.max_len if length is None else length
        if out is None:
            out = np.empty((self.num_kv_heads, L, self.head_dim), np.float32)
        if which == "k" and self.outliers and offsets is None:
            offsets = self.outlier_offsets()

        def fill(h):
            out[h] = self.kv_unit(which, b, h, L, offsets)

        nt = threads or min(16, os.cpu_count() or 1)
        with ThreadPoolExecutor(nt) as ex:
            list(ex.map(fill, range(self.num_kv_heads)))
        return out

    def kv_all(self, which: str) -> np.ndarray:
        """[B][Hkv][L][D] float32 (small workloads only)."""
        out = np.empty((self.batch, self.num_kv_heads, self.max_len, self.head_dim), np.float32)
        for b in range(self.batch):
            self.kv_row(which, b, out=out[b])
        return out


def loguniform_lengths(seed: int, n: int, lo: int, hi: int) -> list:
    """n sequence lengths with log-uniform distribution on [lo, hi] (integers)."""
    u = _rng(seed, S_LENS).random(n)
    lens = np.floor(np.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))).astype(np.int64)
    return [int(v) for v in np.clip(lens, lo, hi)]


def page_permutation(seed: int, n_pages: int) -> np.ndarray:
    """Random placement of n_pages logical pages in a pool of n_pages slots."""
    return _rng(seed, S_PERM).permutation(n_pages).astype(np.int32)


def build_page_table(seq_lens, page_size: int, seed: int):
    """Page table [B][max_pages] int32 (-1 for unused) with pages scattered by a
    seeded permutation of one pool. Returns (table, num_pages)."""
    pages = [(int(L) + page_size - 1) // page_size for L in seq_lens]
    total = int(sum(pages))
    maxp = max(pages) if pages else 0
    perm = page_permutation(seed, total)
    table = np.full((len(seq_lens), max(maxp, 1)), -1, np.int32)
    k = 0
    for b, n in enumerate(pages):
        table[b, :n] = perm[k:k + n]
        k += n
    return table, total


# ---- the named workloads ------------------------------------------------

def tiny_int4() -> Workload:
    """B=1, 1 KV head, 4 query heads, D=128, L=1024, INT4, K channel-wise / V token-wise."""
    return Workload("tiny_int4", 1, 1, 4, 128, [1024], 4, "channel", "token", seed=1)


def mid_int2(k_axis="channel", v_axis="token") -> Workload:
    """B=16, 8 KV x 32 query heads, D=128, L=4096, INT2 (any fold pairing)."""
    return Workload(f"mid_int2_{k_axis[0]}{v_axis[0]}", 16, 8, 32, 128, [4096] * 16, 2,
                    k_axis, v_axis, seed=2)


def headline(bits: int, k_axis="channel", v_axis="token") -> Workload:
    """B=128, 8 KV x 32 query heads, D=128, L=32768, N(0,1) plus K outlier channels.

    Both bit widths draw the same float32 values (seed 3)."""
    return Workload(f"headline_int{bits}_{k_axis[0]}{v_axis[0]}", 128, 8, 32, 128, [32768] * 128,
                    bits, k_axis, v_axis, seed=3, outliers=True)


def tp8_share(bits: int) -> Workload:
    """One GPU's share of the headline under 8-way tensor parallelism: the same
    128 sequences x 32768 tokens, but one KV head and its 4 query heads.
    Own seed (6), same distribution as the headline."""
    return Workload(f"tp8_share_int{bits}", 128, 1, 4, 128, [32768] * 128, bits, "channel", "token",
                    seed=6, outliers=True)


def paged_long(layer: int, n_seq: int = 64, lo: int = 1024, hi: int = 131072) -> Workload:
    """64 sequences, lengths log-uniform in [1K, 128K], 64-token pages in one pool,
    layers alternate INT4, INT2, INT4, INT2; K channel-wise / V token-wise."""
    lens = loguniform_lengths(5, n_seq, lo, hi)
    bits = 4 if layer % 2 == 0 else 2
    return Workload(f"paged_layer{layer}_int{bits}", n_seq, 8, 32, 128, lens, bits, "channel",
                    "token", seed=5, outliers=True, layer=layer, page_size=64)
