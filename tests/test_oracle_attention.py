"""Pins for the float64 attention oracle (CPU only).

Each check ties the oracle to something other than itself: hand-computed closed
forms (tests/golden), identities the definition implies, brute force between
the three-pass and block-loop forms, and a library routine (torch's CPU
scaled_dot_product_attention in float64)."""
import json
import math
import os

import numpy as np
import pytest

from oracle import attention as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def _rand(*shape):
    return RNG.standard_normal(shape)


def test_golden_closed_forms():
    with open(os.path.join(GOLDEN, "softmax_closed_form.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q, k, v = (np.array(c[x]) for x in ("q", "k", "v"))
        for fn in ("naive", "online"):
            if fn == "naive":
                o, lse = A.naive_head(q, k, v, c["scale"], c["causal"])
            else:
                o, lse = A.online_head(q, k, v, c["scale"], 1, c["causal"])
            np.testing.assert_allclose(o, np.array(c["o"]), rtol=0, atol=1e-14, err_msg=c["name"])
            np.testing.assert_allclose(lse, np.array(c["lse"]), rtol=0, atol=1e-14, err_msg=c["name"])


@pytest.mark.parametrize("sk", [1, 5, 100, 128, 129])
@pytest.mark.parametrize("block_c", [1, 7, 16, 64, None])
@pytest.mark.parametrize("causal", [False, True])
def test_naive_equals_online(sk, block_c, causal):
    # pins the rescale direction and that the last partial block is scored
    sq, d = 37, 16
    q, k, v = _rand(sq, d), _rand(sk, d), _rand(sk, d)
    bc = sk if block_c is None else block_c
    o1, l1 = A.naive_head(q, k, v, 0.3, causal)
    o2, l2 = A.online_head(q, k, v, 0.3, bc, causal)
    fin = np.isfinite(l1)
    assert np.array_equal(fin, np.isfinite(l2))
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l2[fin], l1[fin], rtol=1e-12, atol=1e-13)


def test_rows_of_p_sum_to_one():
    q, k, v = _rand(50, 32), _rand(77, 32), _rand(77, 32)
    for causal in (False, True):
        _, _, p = A.naive_head(q, k, v, 0.2, causal, return_p=True)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        assert (p >= 0).all()


def test_single_key_gives_v0():
    q, k, v = _rand(9, 8), _rand(1, 8), _rand(1, 8)
    for method in ("naive", "online"):
        f = A.naive_head if method == "naive" else (lambda *a: A.online_head(*a[:4], 3, *a[4:]))
        o, lse = f(q, k, v, 0.7)
        np.testing.assert_allclose(o, np.repeat(v, 9, axis=0), rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse, 0.7 * (q @ k[0]), rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_v(causal):
    sq, sk, d = 20, 20, 8
    q = _rand(sq, d)
    k = np.repeat(_rand(1, d), sk, axis=0)
    v = _rand(sk, d)
    o, lse = A.naive_head(q, k, v, 0.5, causal)
    cnt = A.valid_key_counts(sq, sk, causal)
    for i in range(sq):
        n = cnt[i]
        np.testing.assert_allclose(o[i], v[:n].mean(axis=0), rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[i], 0.5 * q[i] @ k[0] + math.log(n), rtol=0, atol=1e-12)


def test_causal_row0_gives_v0():
    q, k, v = _rand(16, 8), _rand(16, 8), _rand(16, 8)
    o, lse = A.naive_head(q, k, v, 0.4, True)
    np.testing.assert_allclose(o[0], v[0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0], 0.4 * q[0] @ k[0], rtol=0, atol=1e-14)


@pytest.mark.parametrize("lq,lk", [(16, 16), (7, 30), (30, 7)])
def test_zero_query_gives_mean_and_log_count(lq, lk):
    q, k, v = np.zeros((lq, 4)), _rand(lk, 4), _rand(lk, 4)
    o, lse = A.naive_head(q, k, v, 1.0, True)
    cnt = A.valid_key_counts(lq, lk, True)
    for i in range(lq):
        if cnt[i] == 0:
            assert np.all(o[i] == 0) and lse[i] == -np.inf
        else:
            np.testing.assert_allclose(o[i], v[:cnt[i]].mean(axis=0), rtol=0, atol=1e-13)
            np.testing.assert_allclose(lse[i], math.log(cnt[i]), rtol=0, atol=1e-13)


def test_valid_key_counts_closed_form():
    # square causal: row i sees i + 1 keys; bottom-right alignment for Lq != Lk
    assert list(A.valid_key_counts(5, 5, True)) == [1, 2, 3, 4, 5]
    assert list(A.valid_key_counts(3, 5, True)) == [3, 4, 5]
    assert list(A.valid_key_counts(5, 3, True)) == [0, 0, 1, 2, 3]
    assert list(A.valid_key_counts(4, 6, False)) == [6, 6, 6, 6]


def test_key_shift_invariance():
    q, k, v = _rand(12, 8), _rand(19, 8), _rand(19, 8)
    u = _rand(8)
    o1, l1 = A.naive_head(q, k, v, 0.3, False)
    o2, l2 = A.naive_head(q, k + u, v, 0.3, False)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2 - l1, 0.3 * q @ u, rtol=0, atol=1e-12)


def test_value_affine():
    q, k, v = _rand(12, 8), _rand(19, 8), _rand(19, 8)
    o1, _ = A.naive_head(q, k, v, 0.3, True)
    o2, _ = A.naive_head(q, k, 2.5 * v - 1.25, 0.3, True)
    np.testing.assert_allclose(o2, 2.5 * o1 - 1.25, rtol=0, atol=1e-12)


def test_joint_key_value_permutation():
    q, k, v = _rand(12, 8), _rand(19, 8), _rand(19, 8)
    perm = RNG.permutation(19)
    o1, l1 = A.naive_head(q, k, v, 0.3, False)
    o2, l2 = A.naive_head(q, k[perm], v[perm], 0.3, False)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-13)


def test_large_scores_do_not_overflow():
    q = np.array([[100.0, 0.0], [-100.0, 0.0]])
    k = np.array([[100.0, 0.0], [99.0, 0.0], [-100.0, 0.0]])
    v = np.array([[1.0], [2.0], [3.0]])
    o, lse = A.naive_head(q, k, v, 1.0)      # scores up to +-1e4
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    np.testing.assert_allclose(o[0], [1.0], atol=1e-12)
    np.testing.assert_allclose(lse[0], 1e4, rtol=1e-15)
    o2, lse2 = A.online_head(q, k, v, 1.0, 1)
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, rtol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_against_torch_sdpa_float64(causal):
    torch = pytest.importorskip("torch")
    B, S, H, D = 2, 45, 3, 16
    q, k, v = _rand(B, S, H, D), _rand(B, S, H, D), _rand(B, S, H, D)
    o, lse = A.attention_bshd(q, k, v, 0.25, causal)
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x.transpose(0, 2, 1, 3))) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.25)
    np.testing.assert_allclose(o, ref.numpy().transpose(0, 2, 1, 3), rtol=0, atol=1e-12)
    s = torch.einsum("bhqd,bhkd->bhqk", tq, tk) * 0.25
    if causal:
        s = s.masked_fill(torch.ones(S, S, dtype=torch.bool).triu(1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-12)


def test_row_subset_equals_full():
    B, S, H, D = 1, 64, 2, 8
    q, k, v = _rand(B, S, H, D), _rand(B, S, H, D), _rand(B, S, H, D)
    o, lse = A.attention_bshd(q, k, v, 0.3, True)
    rows = [0, 5, 31, 63]
    o2, lse2 = A.attention_bshd(q, k, v, 0.3, True, rows=rows)
    np.testing.assert_allclose(o2[:, rows], o[:, rows], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse2[:, :, rows], lse[:, :, rows], rtol=0, atol=1e-14)


def test_varlen_and_paged_match_dense():
    lens = [5, 64, 70, 1]
    H, D, page = 2, 8, 16
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    tot = int(cu[-1])
    q, k, v = _rand(tot, H, D), _rand(tot, H, D), _rand(tot, H, D)
    o, lse = A.attention_varlen(q, cu, k, v, cu, 0.35, True)
    for b, n in enumerate(lens):
        sl = slice(cu[b], cu[b + 1])
        od, ld = A.attention_bshd(q[None, sl], k[None, sl], v[None, sl], 0.35, True)
        np.testing.assert_allclose(o[sl], od[0], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[:, sl], ld[0], rtol=0, atol=1e-14)
    # scatter the same keys into shuffled pages and read them back through a table
    pages_per = [(n + page - 1) // page for n in lens]
    perm = RNG.permutation(sum(pages_per))
    kp = np.full((sum(pages_per), page, H, D), np.nan)
    vp = np.full_like(kp, np.nan)
    table = np.full((len(lens), max(pages_per)), -1)
    pos = 0
    for b, n in enumerate(lens):
        for p in range(pages_per[b]):
            phys = perm[pos]
            pos += 1
            table[b, p] = phys
            t0, t1 = p * page, min((p + 1) * page, n)
            kp[phys, :t1 - t0] = k[cu[b] + t0:cu[b] + t1]
            vp[phys, :t1 - t0] = v[cu[b] + t0:cu[b] + t1]
    o2, lse2 = A.attention_varlen(q, cu, kp, vp, cu, 0.35, True, block_table=table, page_size=page)
    np.testing.assert_array_equal(o2, o)
    np.testing.assert_array_equal(lse2, lse)


def test_half_ulp_helper():
    from tests.parity import half_ulp
    assert half_ulp(1.0) == 2.0 ** -8 and half_ulp(3.0) == 2.0 ** -7 and half_ulp(-5.0) == 2.0 ** -6
    assert half_ulp(1.0, "fp16") == 2.0 ** -11


@pytest.mark.parametrize("bounds", [(0, 7, 7, 40, 100), (0, 1, 2, 3, 100), (0, 100)])
def test_merge_of_key_ranges_equals_full_attention(bounds):
    # ranges of keys (one may be empty) attended separately and merged give the
    # attention over all keys: a pin of merge_partials against the definition
    q, k, v = _rand(23, 8), _rand(100, 8), _rand(100, 5)
    parts = [A.naive_head(q, k[lo:hi], v[lo:hi], 0.4) for lo, hi in zip(bounds[:-1], bounds[1:])]
    o, lse = A.merge_partials([p[0] for p in parts], [p[1] for p in parts])
    o_ref, lse_ref = A.naive_head(q, k, v, 0.4)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def test_merge_rows_without_keys():
    # causal rows that see no key in any range stay O = 0, LSE = -inf
    q, k, v = _rand(6, 4), _rand(3, 4), _rand(3, 4)
    o1, l1 = A.naive_head(q, k[:2], v[:2], 1.0, causal=True, lq=6)
    o2, l2 = A.naive_head(q, k[2:], v[2:], 1.0)
    o2[:] = 0.0
    l2[:] = -np.inf
    o, lse = A.merge_partials([o1, o2], [l1, l2])
    np.testing.assert_array_equal(np.isinf(lse), np.isinf(l1))
    np.testing.assert_allclose(o, o1, rtol=0, atol=1e-15)


def test_bias_row_constant_shifts_lse_only():
    # adding c_i to every score of row i leaves the softmax unchanged
    q, k, v = _rand(11, 8), _rand(30, 8), _rand(30, 8)
    c = _rand(11)
    o1, l1 = A.naive_head(q, k, v, 0.3, True)
    o2, l2 = A.naive_head(q, k, v, 0.3, True, bias=np.repeat(c[:, None], 30, axis=1))
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, l1 + c, rtol=0, atol=1e-12)


def test_bias_log_multiplicity_equals_repeated_keys():
    # a bias of ln(m_j) on key j counts that key m_j times: the same attention
    # as the key set with key j written out m_j times
    q, k, v = _rand(9, 6), _rand(12, 6), _rand(12, 6)
    mult = RNG.integers(1, 4, size=12)
    o1, l1 = A.naive_head(q, k, v, 0.5, bias=np.repeat(np.log(mult)[None, :], 9, axis=0))
    o2, l2 = A.naive_head(q, np.repeat(k, mult, axis=0), np.repeat(v, mult, axis=0), 0.5)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)


def test_bias_minus_inf_upper_triangle_is_causal():
    q, k, v = _rand(16, 8), _rand(16, 8), _rand(16, 8)
    mask = np.where(np.triu(np.ones((16, 16)), 1) > 0, -np.inf, 0.0)
    o1, l1 = A.naive_head(q, k, v, 0.4, bias=mask)
    o2, l2 = A.naive_head(q, k, v, 0.4, True)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-14)


def test_bias_against_torch_sdpa_float64():
    torch = pytest.importorskip("torch")
    B, S, H, D = 2, 33, 3, 16
    q, k, v = _rand(B, S, H, D), _rand(B, S, H, D), _rand(B, S, H, D)
    bias = _rand(B, H, S, S)
    o, lse = A.attention_bshd(q, k, v, 0.25, False, bias=bias)
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x.transpose(0, 2, 1, 3))) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(bias), scale=0.25)
    np.testing.assert_allclose(o, ref.numpy().transpose(0, 2, 1, 3), rtol=0, atol=1e-12)
