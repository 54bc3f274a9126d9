"""8-bit integer pieces of the forward pass — oracle (test infrastructure only).

Sources:

* the StreamHPC case study "1 PFLOPS Flash Attention on a single H100",
  section "Our approach": the fused kernel was given an int8 path beside the
  fp8 one (the page gives no further detail of it);
* the "Fused attention kernel" page, section "8-bit forward pass": block
  quantisation (each block of Q, K and V has its own scale instead of one per
  tensor) and incoherent processing (Q and K multiplied by a random-sign
  Hadamard matrix, which cancels in Q K^T).  The int8 path takes both over
  unchanged; only the code format of Q and K differs.

Readings where the pages are silent:

* symmetric int8 codes: scale = amax / 127 in float32 (1 for an all-zero
  block), code = x / scale (float32 division) rounded to nearest with ties to
  even and clamped to [-127, 127]; -128 is never produced, so the code range is
  symmetric and negation is exact;
* a block is 128 consecutive sequence rows of one (batch, head), as for e4m3;
  block_rows = 0 means one scale for the whole tensor;
* decoding is code * scale;
* int8 is the format of Q and K, i.e. of the score product Q K^T, which then
  sums exactly in int32.  V, and the probabilities that multiply it, keep the
  e4m3 format of the 8-bit path: probabilities are fractions of the running
  row maximum, and a fixed-point int8 code (0..127 times the maximum) rounds
  every key below 1/254 of it to zero.  On the outlier workload that loses
  the mass of the many small keys (float64 emulation: RMSE about 1e-1 against
  about 7e-3 with e4m3 probabilities), so the reading that keeps the path
  accurate is int8 scores with an e4m3 output product;
* the rotation and the choice of tensors it applies to (Q and K, not V) are
  those of the e4m3 path.
"""
from __future__ import annotations

import numpy as np

from . import fp8
from .fp8 import rotate

INT8_MAX = 127
BLOCK_ROWS = 128


def int8_encode(y) -> np.ndarray:
    """Already-scaled values y (float32) -> int8 codes: round to nearest, ties
    to even (numpy rint), then clamp to [-127, 127]."""
    y = np.asarray(y, dtype=np.float32).astype(np.float64)
    return np.clip(np.rint(y), -INT8_MAX, INT8_MAX).astype(np.int8)


def int8_decode(codes, scale=1.0) -> np.ndarray:
    return np.asarray(codes, dtype=np.int8).astype(np.float64) * np.asarray(scale, dtype=np.float64)


def scale_from_amax(amax) -> np.ndarray:
    """float32 scale = amax / 127, or 1 for an all-zero block."""
    a = np.asarray(amax, dtype=np.float32)
    return np.where(a > 0, a / np.float32(INT8_MAX), np.float32(1.0)).astype(np.float32)


def quantize(x_bshd, block_rows: int = BLOCK_ROWS):
    """Quantise a [B, S, H, D] tensor to int8 codes.

    block_rows = 128: one scale per (b, h, 128-row block), scales [B, H, nblk];
    block_rows = 0: one scale for the whole tensor, scales [1].
    The code decision is taken in float32.  Returns (codes int8 [B, S, H, D],
    scales float32)."""
    x = np.asarray(x_bshd, dtype=np.float32)
    B, S, H, D = x.shape
    if block_rows == 0:
        scale = scale_from_amax(np.abs(x).max() if x.size else 0.0).reshape(1)
        return int8_encode(x / scale[0]), scale
    nblk = (S + block_rows - 1) // block_rows
    scales = np.ones((B, H, nblk), dtype=np.float32)
    codes = np.zeros(x.shape, dtype=np.int8)
    for i in range(nblk):
        lo, hi = i * block_rows, min((i + 1) * block_rows, S)
        blk = x[:, lo:hi]                                   # [B, rows, H, D]
        sc = scale_from_amax(np.abs(blk).max(axis=(1, 3)))  # [B, H]
        scales[:, :, i] = sc
        codes[:, lo:hi] = int8_encode(blk / sc[:, None, :, None])
    return codes, scales


def dequantize(codes, scales, block_rows: int = BLOCK_ROWS) -> np.ndarray:
    """codes [B, S, H, D] with their scales -> float64 values."""
    vals = np.asarray(codes, dtype=np.int8).astype(np.float64)
    if block_rows == 0:
        return vals * float(np.asarray(scales).reshape(-1)[0])
    B, S, H, D = vals.shape
    row_blk = np.arange(S) // block_rows
    sc = np.asarray(scales, dtype=np.float64)[:, :, row_blk]  # [B, H, S]
    return vals * np.transpose(sc, (0, 2, 1))[..., None]


def quantize_pipeline(q, k, v, signs=None, block_rows: int = BLOCK_ROWS):
    """Optional rotation of Q and K (float64, rounded to float32 before the
    code decision), then int8 quantisation of Q' and K' and e4m3 quantisation
    of V (the 8-bit path's V, unchanged)."""
    if signs is not None:
        q = rotate(q, signs).astype(np.float32)
        k = rotate(k, signs).astype(np.float32)
    q8, qs = quantize(q, block_rows)
    k8, ks = quantize(k, block_rows)
    v8, vs = fp8.quantize(v, block_rows)
    return dict(q8=q8, q_scale=qs, k8=k8, k_scale=ks, v8=v8, v_scale=vs, block_rows=block_rows)


def dequantize_pipeline(qp):
    """The float64 values the quantised path stands for: (Q', K', V)."""
    br = qp["block_rows"]
    return (dequantize(qp["q8"], qp["q_scale"], br), dequantize(qp["k8"], qp["k_scale"], br),
            fp8.dequantize(qp["v8"], qp["v_scale"], br))


def emulate_int8_attention(q, k, v, scale: float, signs=None, block_rows: int = BLOCK_ROWS,
                           causal: bool = False, heads=None, rows=None):
    """Float64 attention of the dequantised inputs (int8 Q', K'; e4m3 V): the
    error that quantising the inputs alone causes (a diagnostic, not the pass
    criterion)."""
    from .attention import attention_bshd
    qd, kd, vd = dequantize_pipeline(quantize_pipeline(q, k, v, signs, block_rows))
    return attention_bshd(qd, kd, vd, scale, causal, heads=heads, rows=rows)
