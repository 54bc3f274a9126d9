"""Seeded synthetic inputs shared by the HIP path, the oracle, the tests and the bench.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  Every generator returns host (numpy) arrays so that the
GPU path and the CPU oracle consume the very same values.

Value recipe (stated once here, used everywhere):

* Q, K, V entries are drawn as float32 N(0, 1) from ``numpy.random.default_rng(seed)``
  in the order Q, K, V, then rounded to bfloat16 with round-to-nearest-even.
  The bf16 values are exactly representable in float32/float64, so a float64
  oracle fed these values computes the exact attention of the GPU's inputs.
* The fp8 accuracy workload adds sparse outliers:
  ``x = N(0,1) + N(0, sigma^2) * Bernoulli(p)`` per entry, with p = 0.001 and
  sigma = 10 (the textbook N(mu, sigma^2) reading of "N(0,100)").
* Varlen lengths are integers uniform in [lo, hi]; page ids are a seeded random
  permutation; the random-sign vector is +-1 with equal probability.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "bf16_round",
    "bf16_bits_to_f32",
    "normal_bf16",
    "outlier_bf16",
    "qkv_normal",
    "qkv_outlier",
    "random_signs",
    "varlen_lengths",
    "paged_layout",
    "Workload",
    "WORKLOADS",
    "seq_sweep_points",
]


# ---------------------------------------------------------------------------
# bf16 rounding (input preparation only)
# ---------------------------------------------------------------------------
def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even) and return the
    16-bit patterns as uint16.  NaN stays NaN (quiet)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rounded = (u + 0x7FFF + lsb) >> 16
    nan = np.isnan(x)
    out = rounded.astype(np.uint16)
    out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 to IEEE half (numpy's cast is round-to-nearest-even)."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16)


# ---------------------------------------------------------------------------
# tensor generators
# ---------------------------------------------------------------------------
def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) float32 draw rounded to bf16; returns float32 holding bf16 values."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return bf16_bits_to_f32(bf16_round(x))


def outlier_bf16(rng: np.random.Generator, shape, sigma: float = 10.0,
                 p: float = 1e-3) -> np.ndarray:
    """N(0,1) + N(0, sigma^2) * Bernoulli(p), drawn in float32, rounded to bf16."""
    base = rng.standard_normal(size=shape, dtype=np.float32)
    big = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(sigma)
    mask = rng.random(size=shape, dtype=np.float32) < np.float32(p)
    x = base + np.where(mask, big, np.float32(0.0))
    return bf16_bits_to_f32(bf16_round(x))


def qkv_normal(seed: int, q_shape, k_shape=None, v_shape=None):
    """Q, K, V ~ N(0,1) in bf16, drawn in the order Q, K, V from one generator."""
    rng = np.random.default_rng(seed)
    k_shape = q_shape if k_shape is None else k_shape
    v_shape = k_shape if v_shape is None else v_shape
    q = normal_bf16(rng, q_shape)
    k = normal_bf16(rng, k_shape)
    v = normal_bf16(rng, v_shape)
    return q, k, v


def qkv_outlier(seed: int, shape, sigma: float = 10.0, p: float = 1e-3):
    rng = np.random.default_rng(seed)
    q = outlier_bf16(rng, shape, sigma, p)
    k = outlier_bf16(rng, shape, sigma, p)
    v = outlier_bf16(rng, shape, sigma, p)
    return q, k, v


def random_signs(seed: int, d: int) -> np.ndarray:
    """Random +-1 diagonal for the incoherent-processing rotation (int8)."""
    rng = np.random.default_rng(seed)
    return np.where(rng.random(d) < 0.5, -1, 1).astype(np.int8)


def varlen_lengths(seed: int, n: int, lo: int, hi: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=n).astype(np.int32)


def cu_seqlens(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    out = np.zeros(len(lengths) + 1, dtype=np.int32)
    out[1:] = np.cumsum(lengths)
    return out


def paged_layout(seed: int, lengths, page_size: int, max_pages_per_seq: int | None = None):
    """Assign each sequence's logical pages to random physical pages.

    Returns (block_table [B, max_pages] int32, num_pages).  Logical page p of
    sequence b lives in physical page ``block_table[b, p]``; entries past the
    sequence's last page are set to -1 (never read)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    pages_per = (lengths + page_size - 1) // page_size
    total = int(pages_per.sum())
    mp = int(pages_per.max()) if max_pages_per_seq is None else int(max_pages_per_seq)
    rng = np.random.default_rng(seed)
    perm = rng.permutation(total).astype(np.int32)
    table = np.full((len(lengths), mp), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(pages_per):
        table[b, :n] = perm[pos:pos + n]
        pos += n
    return table, total


# ---------------------------------------------------------------------------
# the pages' workload shapes
# ---------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    seq_q: int
    seq_k: int
    head_dim: int
    causal: bool
    seed: int
    dtype: str = "bf16"

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def flops(self) -> float:
        f = 4.0 * self.batch * self.heads * self.seq_q * self.seq_k * self.head_dim
        return f / 2 if self.causal else f

    def shapes(self):
        return ((self.batch, self.seq_q, self.heads, self.head_dim),
                (self.batch, self.seq_k, self.heads, self.head_dim))


WORKLOADS = {
    # tiny case: batch 1, 2 heads, 128 x 128, d64, scale 1/8, non-causal
    "tiny": Workload("tiny_b1_h2_s128_d64", 1, 2, 128, 128, 64, False, seed=0),
    # the FlashAttention-3 ablation shape (batch 4, seq 8448, 16 heads, d128)
    "ablation": Workload("ablation_b4_h16_s8448_d128", 4, 16, 8448, 8448, 128, False, seed=1),
    # fp8 accuracy/throughput shape (batch 4, 16 heads, seq 8192, d128)
    "fp8": Workload("fp8_b4_h16_s8192_d128", 4, 16, 8192, 8192, 128, False, seed=3),
}


def seq_sweep_points():
    """16384 tokens per batch: seq in {512..16384}, batch = 16384/seq, hidden
    2048 (head_dim 64/128/256 -> 32/16/8 heads), causal and non-causal."""
    pts = []
    idx = 0
    for d, h in ((64, 32), (128, 16), (256, 8)):
        for s in (512, 1024, 2048, 4096, 8192, 16384):
            for causal in (False, True):
                pts.append(Workload(f"sweep_s{s}_d{d}_{'causal' if causal else 'full'}",
                                    16384 // s, h, s, s, d, causal, seed=2 + idx))
                idx += 1
    return pts


# varlen + paged workload: 32 sequences, lengths U{128..4096}, 32 heads, d128,
# causal, 64-token pages at random physical slots
VARLEN = dict(n_seq=32, lo=128, hi=4096, heads=32, head_dim=128, page_size=64,
              causal=True, seed_lengths=5, seed_pages=6, seed_values=7)

# decoding against a long paged cache: one query row per sequence, every
# sequence 32768 keys in 64-token pages at a seeded permutation of slots
DECODE = dict(n_seq=4, seq_q=1, seq_k=32768, heads=32, head_dim=128, page_size=64, causal=True,
              seed_pages=12, seed_values=13)
