"""Seeded synthetic inputs for the attention forward: the workload shapes and
their random tensors.

This module holds no attention arithmetic. It only describes workloads and
draws their f32 inputs, so that the HIP path and the float64 checker see the
very same arrays. Shapes follow the pages' workloads: whole-sequence causal /
full / cross attention (meganeura attention.wgsl, header: the three variants),
single-token decode over a KV cache (meganeura cached_attention.wgsl, header),
and batched causal prefill continuing a cache from ``start_pos`` (cera
attention_prefill.wgsl, header: constraints and ``params`` block).

Recipe: ``numpy.random.default_rng(1000*cfg + 10*sub + t)`` with t = 1 for Q,
2 for K, 3 for V and 4 for the pick of "heavy" K rows; values are
``standard_normal(dtype=float32)``. Cache rows past the valid window are drawn
the same way (the poison tests overwrite them with NaN).
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

CAUSAL, FULL, CROSS = 0, 1, 2
MODE_NAMES = {CAUSAL: "causal", FULL: "full", CROSS: "cross"}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention call.

    q: [q_seq, num_heads*head_dim]; k, v: [kv_rows, num_kv_heads*head_dim]
    with the first ``kv_len`` rows valid. ``start_pos`` offsets the causal
    window (query i sees keys [0, min(start_pos+i+1, kv_len))).
    """

    name: str
    mode: int
    q_seq: int
    kv_len: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    start_pos: int = 0
    kv_rows: Optional[int] = None  # allocated cache rows (>= kv_len)
    with_lse: bool = True
    heavy_frac: float = 0.0  # fraction of K rows scaled by heavy_gain
    heavy_gain: float = 8.0
    seed_base: int = 0

    @property
    def rows(self) -> int:
        return self.kv_len if self.kv_rows is None else self.kv_rows

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def group(self) -> int:
        return self.num_heads // self.num_kv_heads


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """One-token decode over a KV cache of ``max_seq`` rows; the window is
    [0, min(kv_pos+1, max_seq)) with kv_pos read on the device."""

    name: str
    num_heads: int
    num_kv_heads: int
    head_dim: int
    max_seq: int
    kv_pos_values: tuple
    seed_base: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


# The workloads of the pages, by what they are.
CAUSAL_SMALL = Workload("causal_q32_kv32_h4kv2_d64", CAUSAL, 32, 32, 4, 2, 64,
                        seed_base=1000)
FULL_1K = Workload("full_q1024_kv1024_h8_d64", FULL, 1024, 1024, 8, 8, 64,
                   seed_base=2000)
CROSS_512x2K = Workload("cross_q512_kv2048_h8_d64", CROSS, 512, 2048, 8, 8, 64,
                        seed_base=2010)
DECODE_8K = DecodeWorkload("decode_h32kv8_d128_cache8192", 32, 8, 128, 8192,
                           (127, 1023, 4095, 8191), seed_base=3000)
CONTINUE_512 = Workload("causal_continue_q512_start1536_cache4096_h32kv8_d128",
                        CAUSAL, 512, 2048, 32, 8, 128, start_pos=1536,
                        kv_rows=4096, with_lse=False, seed_base=4000)
CAUSAL_16K = Workload("causal_q16384_kv16384_h32kv8_d128_heavyK", CAUSAL, 16384,
                      16384, 32, 8, 128, heavy_frac=0.01, seed_base=5000)

PREFILL_WORKLOADS = (CAUSAL_SMALL, FULL_1K, CROSS_512x2K, CONTINUE_512, CAUSAL_16K)


def _rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def normal(shape, seed: int) -> np.ndarray:
    return _rng(seed).standard_normal(shape, dtype=np.float32)


def heavy_rows(n_rows: int, frac: float, seed: int) -> np.ndarray:
    """Seeded pick of round(frac*n_rows) distinct row indices (sorted)."""
    count = int(round(frac * n_rows))
    if count == 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(_rng(seed).choice(n_rows, size=count, replace=False))


def make_prefill(w: Workload):
    """Return (q, k, v) float32 arrays for a prefill workload."""
    qd = w.num_heads * w.head_dim
    kvd = w.num_kv_heads * w.head_dim
    q = normal((w.q_seq, qd), w.seed_base + 1)
    k = normal((w.rows, kvd), w.seed_base + 2)
    v = normal((w.rows, kvd), w.seed_base + 3)
    if w.heavy_frac > 0.0:
        idx = heavy_rows(w.kv_len, w.heavy_frac, w.seed_base + 4)
        k[idx] *= np.float32(w.heavy_gain)
    return q, k, v


def make_decode(w: DecodeWorkload):
    """Return (q [1, H*d], k_cache, v_cache [max_seq, Hkv*d]) float32."""
    qd = w.num_heads * w.head_dim
    kvd = w.num_kv_heads * w.head_dim
    q = normal((1, qd), w.seed_base + 1)
    k = normal((w.max_seq, kvd), w.seed_base + 2)
    v = normal((w.max_seq, kvd), w.seed_base + 3)
    return q, k, v


def random_case(seed: int, mode: int, q_seq: int, kv_len: int, num_heads: int,
                num_kv_heads: int, head_dim: int, start_pos: int = 0,
                kv_rows: Optional[int] = None):
    """Small seeded case for parity sweeps; returns (workload, q, k, v)."""
    w = Workload(f"rand{seed}", mode, q_seq, kv_len, num_heads, num_kv_heads,
                 head_dim, start_pos=start_pos, kv_rows=kv_rows,
                 seed_base=seed * 10)
    q, k, v = make_prefill(w)
    return w, q, k, v


def paged_pool(k: np.ndarray, v: np.ndarray, page_size: int, extra_pages: int, seed: int,
               fill=np.nan):
    """Lay a dense cache [max_seq, Hkv*d] out as a paged pool: the row block
    b (page_size rows) goes to page table[b] of a pool of nblk + extra_pages
    pages, with the table a seeded permutation; unused pages and the tail of
    the last page hold `fill`. Returns (k_pool, v_pool [pages, page_size,
    Hkv*d], table int32 [nblk], num_pages)."""
    max_seq, kvd = k.shape
    nblk = -(-max_seq // page_size)
    num_pages = nblk + extra_pages
    table = _rng(seed).permutation(num_pages)[:nblk].astype(np.int32)
    kp = np.full((num_pages, page_size, kvd), fill, np.float32)
    vp = np.full((num_pages, page_size, kvd), fill, np.float32)
    for b in range(nblk):
        lo = b * page_size
        n = min(page_size, max_seq - lo)
        kp[table[b], :n] = k[lo:lo + n]
        vp[table[b], :n] = v[lo:lo + n]
    return kp, vp, table, num_pages
