"""GPU parity of the additive-bias forward (attn_fwd_bias) against the float64
oracle: dense and broadcast bias layouts, both 16-bit types, causal and not,
and -inf bias entries, whose triangle must reproduce the causal kernel bit for
bit."""
import math

import numpy as np
import pytest

import workloads as W
from oracle import attention as OA
from tests.parity import assert_close16, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_attn_fwd_10_amd as A
    return A


def _bias_values(seed, shape, dtype):
    x = np.random.default_rng(seed).standard_normal(shape).astype(np.float32) * 2.0
    if dtype == "bf16":
        return W.bf16_bits_to_f32(W.bf16_round(x))
    return W.f16_round(x).astype(np.float32)


def _run(lib, q, k, v, bias, causal, dtype):
    import torch
    tq, tk, tv = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    tb = lib.pad_bias(to_dev(bias, dtype))
    o, lse = lib.fwd_bias(tq, tk, tv, tb, causal=causal)
    torch.cuda.synchronize()
    return to_host(o), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("bshape", ["full", "per_head_key", "per_batch"])
def test_bias_parity(lib, d, causal, dtype, bshape):
    B, Sq, Sk, H = 2, 200, 333, 3
    q, k, v = W.qkv_normal(1000 + d, (B, Sq, H, d), (B, Sk, H, d))
    if dtype == "fp16":
        q, k, v = (W.f16_round(x).astype(np.float32) for x in (q, k, v))
    shape = {"full": (B, H, Sq, Sk), "per_head_key": (1, H, 1, Sk), "per_batch": (B, 1, Sq, Sk)}[bshape]
    bias = _bias_values(2000 + d, shape, dtype)
    o, lse = _run(lib, q, k, v, bias, causal, dtype)
    o_ref, lse_ref = OA.attention_bshd(q, k, v, 1 / math.sqrt(d), causal, bias=bias)
    assert_close16(o, o_ref, lse, lse_ref, f"bias {bshape} d{d} causal={causal} {dtype}", dtype=dtype)


@pytest.mark.parametrize("d", [64, 128])
def test_minus_inf_triangle_is_the_causal_kernel(lib, d):
    # a -inf bias above the diagonal and no mask gives what the causal kernel
    # gives (up to the one extra rounding of scale * score before the exp2)
    import torch
    B, S, H = 1, 300, 2
    q, k, v = W.qkv_normal(1100 + d, (B, S, H, d), (B, S, H, d))
    tri = np.where(np.triu(np.ones((S, S)), 1) > 0, -np.inf, 0.0).astype(np.float32)[None, None]
    o1, l1 = _run(lib, q, k, v, tri, False, "bf16")
    o2, l2 = lib.fwd(to_dev(q), to_dev(k), to_dev(v), causal=True)
    torch.cuda.synchronize()
    np.testing.assert_allclose(o1, to_host(o2), rtol=2 ** -7, atol=2 ** -12)
    np.testing.assert_allclose(l1, l2.cpu().numpy().astype(np.float64), rtol=0, atol=1e-5)


def test_rows_with_every_key_excluded(lib):
    B, Sq, Sk, H, d = 1, 70, 90, 2, 128
    q, k, v = W.qkv_normal(1200, (B, Sq, H, d), (B, Sk, H, d))
    bias = _bias_values(1201, (B, H, Sq, Sk), "bf16")
    bias[:, :, 5, :] = -np.inf
    bias[:, 1, 33, :] = -np.inf
    o, lse = _run(lib, q, k, v, bias, False, "bf16")
    assert np.all(o[0, 5] == 0.0) and np.all(np.isneginf(lse[0, :, 5]))
    assert np.all(o[0, 33, 1] == 0.0) and np.isneginf(lse[0, 1, 33])
    o_ref, lse_ref = OA.attention_bshd(q, k, v, 1 / math.sqrt(d), False, bias=bias)
    assert_close16(o, o_ref, lse, lse_ref, "excluded rows")
