"""Exact attention forward in float64 — oracle (test infrastructure only).

Sources, all on the "Fused attention kernel" concept page (wikillm):

* Overview: standard attention forms the full score matrix S = Q K^T, the
  probability matrix P = softmax(S) row by row, and the output P V.  The fused
  kernel reaches the same result block by block with a running row maximum and
  row sum.  ``naive_head`` is that three-pass definition; ``online_head`` is the
  block loop.
* Implementation sketch: the loop over key blocks, the running max m, the
  running sum l, the rescale factor alpha = exp(m_old - m_new) applied to both l
  and the output, the single normalisation o / l at the end and lse = m + log l.
* The two notes under the sketch: the rescale is exp(old max - new max) (not its
  inverse) and every key block is scored, including a last partial block.

Readings where the pages are silent (each also listed in the design notes):

* the scores are scaled: s_ij = scale * <q_i, k_j> (the pages' "scaled
  dot-product"); the returned lse is the natural log of sum_j exp(s_ij);
* causal masking keeps key j for query i iff j <= i + (Lk - Lq) (bottom-right
  alignment; identical to j <= i when Lq == Lk);
* a query row with no allowed key has o = 0 and lse = -inf;
* masked keys never contribute, whatever their K/V memory holds.

Layouts: dense tensors are [B, S, H, D]; the LSE is [B, H, Sq].  Varlen tensors
are packed [total, H, D] with int32 prefix sums ``cu_seqlens``; their LSE is
[H, total_q].
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = -math.inf


# ---------------------------------------------------------------------------
# masks
# ---------------------------------------------------------------------------
def allowed(rows, lq: int, lk: int, causal: bool) -> np.ndarray:
    """Boolean [len(rows), lk]: may query row i attend to key j?"""
    rows = np.asarray(rows, dtype=np.int64)
    j = np.arange(lk, dtype=np.int64)[None, :]
    ok = np.ones((len(rows), lk), dtype=bool)
    if causal:
        ok &= j <= rows[:, None] + (lk - lq)
    return ok


def valid_key_counts(lq: int, lk: int, causal: bool) -> np.ndarray:
    """|A_i| for every query row: the number of keys row i may attend to."""
    return allowed(np.arange(lq), lq, lk, causal).sum(axis=1).astype(np.int64)


# ---------------------------------------------------------------------------
# one head, three passes (the plain definition)
# ---------------------------------------------------------------------------
def naive_head(q, k, v, scale: float, causal: bool = False, rows=None, lq=None,
               return_p: bool = False, bias=None):
    """Scores, then row max, then row sum, then P and O = P V.

    q: [n, D] query rows (their indices in the sequence are ``rows``, default
    0..n-1, and the sequence has ``lq`` rows, default n); k, v: [Lk, D].
    ``bias`` [n, Lk] (optional) is added to the scaled scores before the mask
    and the softmax: s = scale <q, k> + bias (the additive-bias variant the
    pages list; -inf entries exclude keys).
    Returns (o [n, D], lse [n]) and P [n, Lk] when ``return_p``."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, lk = q.shape[0], k.shape[0]
    rows = np.arange(n) if rows is None else np.asarray(rows)
    lq = n if lq is None else lq
    # pass 1: scaled scores (plus the bias), masked
    s = scale * (q @ k.T)
    if bias is not None:
        s = s + np.asarray(bias, dtype=np.float64)
    ok = allowed(rows, lq, lk, causal) & ~np.isneginf(s)
    s = np.where(ok, s, NEG_INF)
    # pass 2: row max and row sum of exp(s - max)
    m = s.max(axis=1) if lk > 0 else np.full(n, NEG_INF)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe[:, None])
    l = e.sum(axis=1)
    # pass 3: probabilities and output
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.where(empty[:, None], 0.0, e / np.where(empty, 1.0, l)[:, None])
    o = p @ v
    lse = np.where(empty, NEG_INF, m_safe + np.log(np.where(empty, 1.0, l)))
    if return_p:
        return o, lse, p
    return o, lse


# ---------------------------------------------------------------------------
# one head, block by block with a running max and sum (the page's loop)
# ---------------------------------------------------------------------------
def online_head(q, k, v, scale: float, block_c: int, causal: bool = False,
                rows=None, lq=None):
    """The Implementation-sketch loop in float64, one query block ``q``.

    Every key block is visited, the last one possibly partial.  With a causal
    mask a row may have seen no allowed key yet (m = -inf); then the exponent
    offset is taken as 0 so that exp(-inf - (-inf)) never arises."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, d = q.shape
    lk = k.shape[0]
    rows = np.arange(n) if rows is None else np.asarray(rows)
    lq = n if lq is None else lq
    o = np.zeros((n, v.shape[1]))
    m = np.full(n, NEG_INF)
    l = np.zeros(n)
    for j in range(math.ceil(lk / block_c)):
        lo, hi = j * block_c, min((j + 1) * block_c, lk)
        s = scale * (q @ k[lo:hi].T)
        ok = allowed(rows, lq, lk, causal)[:, lo:hi]
        s = np.where(ok, s, NEG_INF)
        m_new = np.maximum(m, s.max(axis=1))
        m_use = np.where(np.isfinite(m_new), m_new, 0.0)
        alpha = np.exp(m - m_use)            # exp(old max - new max)
        p = np.exp(s - m_use[:, None])
        l = alpha * l + p.sum(axis=1)
        o = alpha[:, None] * o + p @ v[lo:hi]
        m = m_new
    empty = l == 0.0
    o = np.where(empty[:, None], 0.0, o / np.where(empty, 1.0, l)[:, None])
    lse = np.where(empty, NEG_INF, m + np.log(np.where(empty, 1.0, l)))
    return o, lse


# ---------------------------------------------------------------------------
# batched layouts
# ---------------------------------------------------------------------------
def attention_bshd(q, k, v, scale: float, causal: bool = False, heads=None,
                   rows=None, method: str = "naive", block_c: int = 64, bias=None):
    """Dense [B, S, H, D] attention.  ``heads`` limits the work to a list of
    (b, h) pairs and ``rows`` to a list of query rows; outputs not computed are
    NaN.  ``bias`` (naive method only) broadcasts to [B, H, Sq, Sk] and is added
    to the scaled scores.  Returns (o [B, Sq, H, D], lse [B, H, Sq])."""
    B, sq, H, D = q.shape
    lk = k.shape[1]
    o = np.full((B, sq, H, v.shape[3]), np.nan)
    lse = np.full((B, H, sq), np.nan)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    ridx = np.arange(sq) if rows is None else np.asarray(rows)
    for b, h in pairs:
        qq = np.asarray(q[b, ridx, h, :], dtype=np.float64)
        kk = np.asarray(k[b, :, h, :], dtype=np.float64)
        vv = np.asarray(v[b, :, h, :], dtype=np.float64)
        if method == "naive":
            bb = None
            if bias is not None:
                bb = np.broadcast_to(bias, (B, H, sq, lk))[b, h][ridx]
            oo, ll = naive_head(qq, kk, vv, scale, causal, rows=ridx, lq=sq, bias=bb)
        else:
            oo, ll = online_head(qq, kk, vv, scale, block_c, causal, rows=ridx, lq=sq)
        o[b, ridx, h, :] = oo
        lse[b, h, ridx] = ll
    return o, lse


def gather_paged(pages, block_table_row, length: int, page_size: int):
    """Rebuild one sequence's contiguous [length, H, D] K or V from a paged
    cache [num_pages, page_size, H, D]: token t lives in physical page
    block_table_row[t // page_size] at slot t % page_size."""
    t = np.arange(length)
    phys = np.asarray(block_table_row, dtype=np.int64)[t // page_size]
    return pages[phys, t % page_size]


def attention_varlen(q, cu_q, k, v, cu_k, scale: float, causal: bool = False,
                     block_table=None, page_size: int = 0, seqs=None):
    """Packed variable-length attention.

    q: [total_q, H, D]; cu_q, cu_k: int prefix sums [B+1].  Without a block
    table k, v are packed [total_k, H, D]; with one they are paged caches
    [num_pages, page_size, H, D] and sequence b's key t is read through
    block_table[b].  Returns (o [total_q, H, D], lse [H, total_q]); sequences
    not listed in ``seqs`` are left NaN."""
    total_q, H, D = q.shape
    o = np.full((total_q, H, v.shape[-1]), np.nan)
    lse = np.full((H, total_q), np.nan)
    nb = len(cu_q) - 1
    for b in (range(nb) if seqs is None else seqs):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        lk = int(cu_k[b + 1]) - int(cu_k[b])
        if block_table is None:
            kb = k[int(cu_k[b]):int(cu_k[b]) + lk]
            vb = v[int(cu_k[b]):int(cu_k[b]) + lk]
        else:
            kb = gather_paged(k, block_table[b], lk, page_size)
            vb = gather_paged(v, block_table[b], lk, page_size)
        for h in range(H):
            oo, ll = naive_head(q[q0:q1, h], kb[:, h], vb[:, h], scale, causal)
            o[q0:q1, h] = oo
            lse[h, q0:q1] = ll
    return o, lse


def merge_partials(outs, lses):
    """Combine the results of disjoint key ranges of the same query rows.

    ``outs[s]`` [rows, Dv] is the normalised output and ``lses[s]`` [rows] the
    natural-log logsumexp of range s (-inf: the range held no allowed key).
    The running max and sum of [FAK Implementation sketch] make this exact:
    with L = ln sum_s exp(L_s), the merged output is sum_s exp(L_s - L) O_s and
    the merged logsumexp is L.  A row no range saw gets O = 0, L = -inf."""
    L = np.stack([np.asarray(x, dtype=np.float64) for x in lses])      # [S, rows]
    O = np.stack([np.asarray(x, dtype=np.float64) for x in outs])      # [S, rows, Dv]
    m = L.max(axis=0)
    seen = np.isfinite(m)
    shift = np.where(seen, m, 0.0)
    w = np.where(np.isfinite(L), np.exp(L - shift[None, :]), 0.0)      # [S, rows]
    wsum = w.sum(axis=0)
    o = np.einsum("sr,srd->rd", w, O)
    o = np.where(seen[:, None], o / np.where(seen, wsum, 1.0)[:, None], 0.0)
    lse = np.where(seen, shift + np.log(np.where(seen, wsum, 1.0)), -np.inf)
    return o, lse
