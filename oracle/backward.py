"""Gradients of the attention forward in float64 — oracle (test infrastructure only).

Sources: the FlashAttention-3 summary page (Key Results: the method has a
backward pass, reported faster than FlashAttention-2's) and the "Fused
attention kernel" page (When to use which: the backward pass follows the same
pattern).  Neither page writes the backward out, so this module is the plain
definition: the gradients, by the chain rule, of

    s_ij = scale <q_i, k_j>   (masked to -inf outside the allowed set A_i),
    P    = softmax over each row of s,
    O    = P V,

with respect to Q, K and V, given the upstream gradient dO.  Written out:

    dV   = P^T dO
    dP   = dO V^T
    dS   = P * (dP - rowsum(P * dP))          (softmax's Jacobian, row by row)
    dQ   = scale dS K
    dK   = scale dS^T Q

Readings where the pages are silent:

* the masks, the scale and the empty-row convention are those of the forward
  (``oracle.attention``); a row with no allowed key has P = 0 and passes no
  gradient;
* the gradients are of the exact (unquantised) forward: the 16-bit inputs are
  taken as exact values.

Layouts: [B, S, H, D] for every tensor.
"""
from __future__ import annotations

import numpy as np

from .attention import naive_head


def backward_head(q, k, v, do, scale: float, causal: bool = False):
    """One (batch, head): q, do [Lq, D]; k, v [Lk, D].  Returns (dq, dk, dv)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    _, _, p = naive_head(q, k, v, scale, causal, return_p=True)
    dv = p.T @ do
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def backward_bshd(q, k, v, do, scale: float, causal: bool = False, heads=None):
    """Dense [B, S, H, D] gradients; ``heads`` limits the work to a list of
    (b, h) pairs (gradients not computed are NaN)."""
    B, Lq, H, D = q.shape
    Lk = k.shape[1]
    dq = np.full((B, Lq, H, D), np.nan)
    dk = np.full((B, Lk, H, D), np.nan)
    dv = np.full((B, Lk, H, v.shape[3]), np.nan)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for b, h in pairs:
        g = backward_head(q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h], scale, causal)
        dq[b, :, h], dk[b, :, h], dv[b, :, h] = g
    return dq, dk, dv
