"""8-bit pieces of the forward pass — oracle (test infrastructure only).

Sources: the "Fused attention kernel" page (wikillm), section "8-bit forward
pass (FP8, Hopper)": the e4m3 format, block quantisation (each block of Q, K and
V gets its own scale instead of one scale per tensor) and incoherent processing
(Q and K multiplied by an orthogonal matrix built from a random sign diagonal
and a Hadamard matrix, which cancels in Q K^T).  The same section gives the
accuracy protocol: RMSE against a float64 reference on synthetic inputs with
0.1 % outliers, block quantisation + rotation against a per-tensor baseline.

Readings where the pages are silent:

* e4m3 is the OCP E4M3FN encoding (bias 7, no infinities, 0x7F/0xFF are NaN,
  largest finite 448), the one the gfx950 matrix cores consume;
* rounding is to nearest, ties to even, saturating at +-448;
* a block is 128 consecutive sequence rows of one (batch, head); the scale of a
  block is amax / 448 computed in float32 (1 when amax = 0), and a value is
  coded as e4m3(x / scale) with the division in float32 — the quantised code is
  a float decision, so it is taken in the kernel's precision (float32);
* the power-of-two form (the input form of the forward that applies block
  scales inside its matrix-core products): the section fixes no scale format,
  and a power of two is a shared exponent.  Its scale is the smallest power of
  two at or above amax / 448 (that quotient rounded to float32), at least
  2^-126 (1 when amax = 0), so x / scale is exact; Q is first multiplied by
  the softmax scale times log2(e) (float32 products, the kernel's precision
  for the code decision), so that the scores come out as base-2 exponents —
  any per-block scale multiplies Q K^T exactly, so attention is unchanged
  once that factor is divided out of the dequantised Q;
* the rotation is M = diag(sigma) H_D / sqrt(D) with H_D the Sylvester
  Hadamard matrix, applied along the head dimension to Q and K only;
* V is block-quantised without rotation.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0
E4M3_NAN = 0x7F
BLOCK_ROWS = 128


# ---------------------------------------------------------------------------
# e4m3fn codec, from the format definition
# ---------------------------------------------------------------------------
def e4m3_decode(codes) -> np.ndarray:
    """uint8 codes -> float64.  s eeee mmm: exponent bias 7; exponent field 0
    is subnormal (m/8 * 2^-6); 0x7F / 0xFF are NaN; there is no infinity."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    val = np.where(e == 0, sub, normal) * sign
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def e4m3_encode(x) -> np.ndarray:
    """Round to the nearest e4m3fn value (ties to even), saturating at +-448.
    NaN -> 0x7F.  Works in float64; every step below is exact except the one
    rounding."""
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x)
    a = np.abs(x)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, a)
    a = np.minimum(a, E4M3_MAX)
    # exponent of the binade holding a; below 2^-6 the spacing is fixed (subnormals)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)
    quantum = np.exp2(e - 3.0)                  # 3 mantissa bits
    qv = np.rint(a / quantum) * quantum          # numpy rint: ties to even
    qv = np.minimum(qv, E4M3_MAX)
    # encode the rounded magnitude
    with np.errstate(divide="ignore"):
        e2 = np.floor(np.log2(np.where(qv > 0, qv, 1.0)))
    is_norm = qv >= 2.0 ** -6
    e2 = np.where(is_norm, e2, -6.0)
    mant_norm = np.rint(qv / np.exp2(e2) * 8.0 - 8.0)
    mant_sub = np.rint(qv / 2.0 ** -9)
    code = np.where(is_norm, ((e2 + 7.0) * 8.0 + mant_norm), mant_sub).astype(np.int64)
    code = np.where(sign, code | 0x80, code)
    code = np.where(nan, E4M3_NAN, code)
    return code.astype(np.uint8)


def e4m3_ulp(x) -> np.ndarray:
    """Spacing of e4m3 values at magnitude |x| (for tolerance statements):
    2^(e-3) in the binade [2^e, 2^(e+1)) for e >= -6, and the subnormal
    spacing 2^-9 below 2^-6, zero included."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 2.0 ** -9)))
    e = np.maximum(e, -6.0)
    return np.exp2(e - 3.0)


# ---------------------------------------------------------------------------
# rotation: random sign diagonal times Hadamard
# ---------------------------------------------------------------------------
def sylvester_hadamard(d: int) -> np.ndarray:
    """H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]] (integer entries +-1)."""
    if d < 1 or d & (d - 1):
        raise ValueError("Hadamard order must be a power of two")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def fwht(x: np.ndarray) -> np.ndarray:
    """Fast Walsh-Hadamard transform along the last axis (unnormalised):
    returns x @ H_D for the Sylvester H_D, by log2(D) butterfly stages."""
    y = np.array(x, dtype=np.float64, copy=True)
    d = y.shape[-1]
    h = 1
    while h < d:
        y = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        y = y.reshape(y.shape[:-3] + (d,))
        h *= 2
    return y


def rotation_matrix(signs) -> np.ndarray:
    """M = diag(signs) @ H_D / sqrt(D); orthogonal."""
    s = np.asarray(signs, dtype=np.float64)
    d = s.shape[0]
    return s[:, None] * sylvester_hadamard(d) / math.sqrt(d)


def rotate(x, signs) -> np.ndarray:
    """x @ M along the last axis, i.e. fwht(x * signs) / sqrt(D), in float64."""
    s = np.asarray(signs, dtype=np.float64)
    return fwht(np.asarray(x, dtype=np.float64) * s) / math.sqrt(s.shape[0])


# ---------------------------------------------------------------------------
# quantisers
# ---------------------------------------------------------------------------
def scale_from_amax(amax) -> np.ndarray:
    """float32 scale = amax / 448, or 1 for an all-zero block."""
    a = np.asarray(amax, dtype=np.float32)
    return np.where(a > 0, a / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)


def quantize(x_bshd, block_rows: int = BLOCK_ROWS):
    """Quantise a [B, S, H, D] tensor to e4m3 codes.

    block_rows = 128: one scale per (b, h, 128-row block), scales [B, H, nblk];
    block_rows = 0: one scale for the whole tensor, scales [1].
    The input is first taken to float32 (the kernel's precision for the code
    decision).  Returns (codes uint8 [B, S, H, D], scales float32)."""
    x = np.asarray(x_bshd, dtype=np.float32)
    B, S, H, D = x.shape
    if block_rows == 0:
        scale = scale_from_amax(np.abs(x).max() if x.size else 0.0).reshape(1)
        codes = e4m3_encode((x / scale[0]).astype(np.float32))
        return codes, scale
    nblk = (S + block_rows - 1) // block_rows
    scales = np.ones((B, H, nblk), dtype=np.float32)
    codes = np.zeros(x.shape, dtype=np.uint8)
    for i in range(nblk):
        lo, hi = i * block_rows, min((i + 1) * block_rows, S)
        blk = x[:, lo:hi]                                   # [B, rows, H, D]
        amax = np.abs(blk).max(axis=(1, 3))                 # [B, H]
        sc = scale_from_amax(amax)
        scales[:, :, i] = sc
        codes[:, lo:hi] = e4m3_encode((blk / sc[:, None, :, None]).astype(np.float32))
    return codes, scales


def scale_pow2_from_amax(amax) -> np.ndarray:
    """Power-of-two form: the smallest power of two >= float32(amax / 448), at
    least 2^-126; 1 for an all-zero block."""
    a = np.asarray(amax, dtype=np.float32)
    t = (a / np.float32(E4M3_MAX)).astype(np.float32)
    mant, ex = np.frexp(t.astype(np.float64))          # t = mant * 2^ex, mant in [0.5, 1)
    e = np.where(mant == 0.5, ex - 1, ex)               # t a power of two: itself
    e = np.where(t > 0, np.maximum(e, -126), -126)      # (a quotient that underflows to 0 too)
    return np.where(a > 0, np.exp2(e.astype(np.float64)), 1.0).astype(np.float32)


def quantize_pow2(x_bshd, block_rows: int = BLOCK_ROWS, premul: float = 1.0):
    """The power-of-two form of quantize: x taken to float32 and multiplied by
    float32(premul) in float32, then scales from scale_pow2_from_amax and codes
    e4m3(x / scale) (an exact division).  Returns (codes, scales) shaped as
    quantize's."""
    x = np.asarray(x_bshd, dtype=np.float32) * np.float32(premul)
    B, S, H, D = x.shape
    if block_rows == 0:
        scale = scale_pow2_from_amax(np.abs(x).max() if x.size else 0.0).reshape(1)
        return e4m3_encode(x.astype(np.float64) / float(scale[0])), scale
    nblk = (S + block_rows - 1) // block_rows
    scales = np.ones((B, H, nblk), dtype=np.float32)
    codes = np.zeros(x.shape, dtype=np.uint8)
    for i in range(nblk):
        lo, hi = i * block_rows, min((i + 1) * block_rows, S)
        blk = x[:, lo:hi]
        sc = scale_pow2_from_amax(np.abs(blk).max(axis=(1, 3)))
        scales[:, :, i] = sc
        codes[:, lo:hi] = e4m3_encode(blk.astype(np.float64) / sc[:, None, :, None].astype(np.float64))
    return codes, scales


def dequantize(codes, scales, block_rows: int = BLOCK_ROWS) -> np.ndarray:
    """codes [B, S, H, D] with their scales -> float64 values."""
    vals = e4m3_decode(codes)
    if block_rows == 0:
        return vals * float(scales.reshape(-1)[0])
    B, S, H, D = vals.shape
    row_blk = np.arange(S) // block_rows                    # [S]
    sc = np.asarray(scales, dtype=np.float64)[:, :, row_blk]  # [B, H, S]
    return vals * np.transpose(sc, (0, 2, 1))[..., None]


def quantize_pipeline(q, k, v, signs=None, block_rows: int = BLOCK_ROWS):
    """The 8-bit prologue: optional rotation of Q and K, then quantisation of
    Q', K' and V.  The rotation is evaluated in float64 and rounded to float32
    before the code decision.  Returns a dict of codes and scales."""
    if signs is not None:
        q = rotate(q, signs).astype(np.float32)
        k = rotate(k, signs).astype(np.float32)
    q8, qs = quantize(q, block_rows)
    k8, ks = quantize(k, block_rows)
    v8, vs = quantize(v, block_rows)
    return dict(q8=q8, q_scale=qs, k8=k8, k_scale=ks, v8=v8, v_scale=vs,
                block_rows=block_rows)


LOG2E = 1.4426950408889634


def quantize_pipeline_pow2(q, k, v, signs=None, block_rows: int = BLOCK_ROWS, *, scale: float):
    """quantize_pipeline in the power-of-two form: Q' multiplied by the softmax
    scale times log2(e) before its quantisation.  The dict also holds that
    factor as q_premul."""
    if signs is not None:
        q = rotate(q, signs).astype(np.float32)
        k = rotate(k, signs).astype(np.float32)
    pm = float(scale) * LOG2E
    q8, qs = quantize_pow2(q, block_rows, pm)
    k8, ks = quantize_pow2(k, block_rows)
    v8, vs = quantize_pow2(v, block_rows)
    return dict(q8=q8, q_scale=qs, k8=k8, k_scale=ks, v8=v8, v_scale=vs,
                block_rows=block_rows, q_premul=pm)


def dequantize_pipeline(qp):
    """Float64 Q', K', V of a quantize_pipeline(_pow2) result, a Q premul
    divided out (so that the softmax scale applies to Q' K'^T again)."""
    br = qp["block_rows"]
    qd = dequantize(qp["q8"], qp["q_scale"], br) / qp.get("q_premul", 1.0)
    return qd, dequantize(qp["k8"], qp["k_scale"], br), dequantize(qp["v8"], qp["v_scale"], br)


def emulate_fp8_attention(q, k, v, scale: float, signs=None, block_rows: int = BLOCK_ROWS,
                          causal: bool = False, heads=None, rows=None):
    """Float64 attention of the dequantised 8-bit inputs (the rotation cancels
    in Q K^T, so the rotated Q', K' are used as they are).  This predicts the
    error that quantising Q, K and V alone causes; it is a diagnostic, not the
    pass criterion."""
    from .attention import attention_bshd
    qp = quantize_pipeline(q, k, v, signs, block_rows)
    qd = dequantize(qp["q8"], qp["q_scale"], block_rows)
    kd = dequantize(qp["k8"], qp["k_scale"], block_rows)
    vd = dequantize(qp["v8"], qp["v_scale"], block_rows)
    return attention_bshd(qd, kd, vd, scale, causal, heads=heads, rows=rows)


def rmse(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.sqrt(np.mean((a - b) ** 2)))
