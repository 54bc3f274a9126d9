"""Pins for the float64 backward oracle (CPU only): central finite differences
of the forward (brute force, independent of the written-out chain rule),
torch's autograd in float64 through a library attention, and identities the
gradients must satisfy exactly."""
import math

import numpy as np
import pytest

from oracle import attention as A
from oracle import backward as G


def _loss(q, k, v, w, scale, causal):
    o, _ = A.naive_head(q, k, v, scale, causal)
    return float((o * w).sum())


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lq,lk", [(4, 5), (5, 3), (3, 3), (1, 6)])
def test_finite_differences(causal, lq, lk):
    rng = np.random.default_rng(lq * 10 + lk + causal)
    d = 3
    q, k, v, w = (rng.standard_normal(s) for s in ((lq, d), (lk, d), (lk, d), (lq, d)))
    scale = 0.7
    dq, dk, dv = G.backward_head(q, k, v, w, scale, causal)
    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            fp = _loss(q, k, v, w, scale, causal)
            x[idx] = old - h
            fm = _loss(q, k, v, w, scale, causal)
            x[idx] = old
            num[idx] = (fp - fm) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("causal", [False, True])
def test_torch_autograd_float64(causal):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    lq, lk, d = 9, 13, 8
    q, k, v, w = (rng.standard_normal(s) for s in ((lq, d), (lk, d), (lk, d), (lq, d)))
    scale = 1 / math.sqrt(d)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    mask = None
    if causal:   # bottom-right alignment: key j allowed for query i iff j <= i + lk - lq
        mask = torch.ones(lq, lk, dtype=torch.bool).tril(diagonal=lk - lq)
    o = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None], attn_mask=mask,
                                                         scale=scale)[0]
    (o * torch.tensor(w)).sum().backward()
    dq, dk, dv = G.backward_head(q, k, v, w, scale, causal)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_identities(causal):
    """Shifting every key by one vector shifts each row's scores by a constant,
    so the key gradients sum to zero; the rows of P sum to one, so the value
    gradients sum to the sum of dO over rows that see a key."""
    rng = np.random.default_rng(8)
    lq, lk, d = 20, 17, 6
    q, k, v, w = (rng.standard_normal(s) for s in ((lq, d), (lk, d), (lk, d), (lq, d)))
    dq, dk, dv = G.backward_head(q, k, v, w, 0.4, causal)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    seen = A.valid_key_counts(lq, lk, causal) > 0
    np.testing.assert_allclose(dv.sum(axis=0), w[seen].sum(axis=0), rtol=1e-12, atol=1e-12)
    # rows with no key (causal, lq > lk) pass no gradient to q
    if causal:
        assert (dq[~seen] == 0).all() and (~seen).any()


def test_single_key():
    """One key: P = 1 everywhere, O = V[0]: dQ = dK = 0 and dV = sum of dO."""
    rng = np.random.default_rng(9)
    q, k, v, w = (rng.standard_normal(s) for s in ((6, 4), (1, 4), (1, 4), (6, 4)))
    dq, dk, dv = G.backward_head(q, k, v, w, 0.5)
    assert np.abs(dq).max() < 1e-14 and np.abs(dk).max() < 1e-14
    np.testing.assert_allclose(dv[0], w.sum(axis=0), rtol=1e-14)


def test_scale_moves_between_q_and_scale():
    """(c q, scale / c) gives the same forward, so dQ scales by 1/c and dK, dV
    are unchanged."""
    rng = np.random.default_rng(10)
    q, k, v, w = (rng.standard_normal(s) for s in ((7, 5), (9, 5), (9, 5), (7, 5)))
    g1 = G.backward_head(q, k, v, w, 0.3)
    g2 = G.backward_head(2.5 * q, k, v, w, 0.3 / 2.5)
    np.testing.assert_allclose(g2[0] * 2.5, g1[0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(g2[1], g1[1], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(g2[2], g1[2], rtol=1e-12, atol=1e-14)


def test_bshd_layout_matches_heads():
    rng = np.random.default_rng(11)
    q, k, v, w = (rng.standard_normal((2, 6, 3, 4)) for _ in range(4))
    dq, dk, dv = G.backward_bshd(q, k, v, w, 0.5, True)
    for b in range(2):
        for h in range(3):
            g = G.backward_head(q[b, :, h], k[b, :, h], v[b, :, h], w[b, :, h], 0.5, True)
            np.testing.assert_array_equal(dq[b, :, h], g[0])
            np.testing.assert_array_equal(dk[b, :, h], g[1])
            np.testing.assert_array_equal(dv[b, :, h], g[2])
