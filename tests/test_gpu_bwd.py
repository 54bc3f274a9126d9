"""GPU parity of the backward pass (attn_bwd) against the float64 oracle
gradients (oracle.backward).

The forward's outputs the backward consumes (O rounded to the 16-bit type, the
fp32 logsumexp) come from the oracle, so the comparison isolates the backward;
one case chains the GPU forward into it.

Tolerance, from the arithmetic: the kernels round P and dS to the 16-bit type
before their matrix products (relative error <= 2^-9 per element for bf16),
form delta from the rounded O, accumulate in fp32 and round the gradients to
the 16-bit type once.  Errors of that size average over the summed keys or
queries, so per gradient tensor the relative RMSE ||G - G_ref|| / ||G_ref|| is
bounded by 1e-2 (about 3x the expected 2^-9 scale) and every element by
5e-2 * max|G_ref|."""
import math

import numpy as np
import pytest

import workloads as W
from oracle import attention as OA
from oracle import backward as OB
from tests.parity import to_dev

pytestmark = pytest.mark.gpu

REL_RMSE = 1e-2
REL_MAX = 5e-2


@pytest.fixture(scope="module")
def lib():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_attn_fwd_10_amd as A
    return A


def _inputs(seed, B, Sq, Sk, H, D):
    q, k, v = W.qkv_normal(seed, (B, Sq, H, D), (B, Sk, H, D))
    do, _, _ = W.qkv_normal(seed + 1000, (B, Sq, H, D))
    return q, k, v, do


def _run_bwd(lib, q, k, v, do, scale, causal, dtype="bf16", o=None, lse=None):
    import torch
    if o is None:
        o, lse = OA.attention_bshd(q, k, v, scale, causal)
        o = np.nan_to_num(o)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    to = torch.from_numpy(np.ascontiguousarray(o, dtype=np.float32)).to(tdt).cuda() if isinstance(o, np.ndarray) else o
    tl = torch.from_numpy(np.ascontiguousarray(lse, dtype=np.float32)).cuda() if isinstance(lse, np.ndarray) else lse
    dq, dk, dv = lib.bwd(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), to, tl, to_dev(do, dtype), scale,
                         causal)
    torch.cuda.synchronize()
    return tuple(t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv))


def _check(got, ref, what):
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert not np.isnan(g).any(), f"{what} {name}: NaN"
        nr = np.sqrt(np.mean(r * r))
        if nr == 0:
            assert np.abs(g).max() == 0, f"{what} {name}: expected zeros"
            continue
        rel = np.sqrt(np.mean((g - r) ** 2)) / nr
        mx = np.abs(g - r).max() / np.abs(r).max()
        assert rel <= REL_RMSE and mx <= REL_MAX, f"{what} {name}: rel rmse {rel:.2e}, rel max {mx:.2e}"


def _rounded(x, dtype):
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(tdt).float().numpy().astype(np.float64)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,Sq,Sk,H,D", [(1, 128, 128, 2, 64), (2, 200, 333, 2, 128), (1, 333, 200, 2, 128),
                                         (1, 1, 1, 1, 64), (1, 64, 300, 2, 128), (2, 300, 64, 1, 64),
                                         (1, 257, 257, 2, 128), (1, 130, 1000, 1, 128)])
def test_bwd_vs_oracle(lib, causal, B, Sq, Sk, H, D):
    q, k, v, do = _inputs(300 + Sq + Sk + D, B, Sq, Sk, H, D)
    scale = 1 / math.sqrt(D)
    ref = OB.backward_bshd(q, k, v, do, scale, causal)
    got = _run_bwd(lib, q, k, v, do, scale, causal)
    _check(got, ref, f"B{B} Sq{Sq} Sk{Sk} H{H} D{D} causal={causal}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_fp16(lib, D, causal):
    q, k, v, do = _inputs(400 + D, 1, 190, 230, 2, D)
    q, k, v, do = (_rounded(x, "fp16") for x in (q, k, v, do))
    scale = 1 / math.sqrt(D)
    ref = OB.backward_bshd(q, k, v, do, scale, causal)
    got = _run_bwd(lib, q, k, v, do, scale, causal, dtype="fp16")
    _check(got, ref, f"fp16 D{D} causal={causal}")


def test_bwd_chained_after_gpu_forward(lib):
    """The GPU forward's own O and LSE feed the GPU backward."""
    import torch
    q, k, v, do = _inputs(500, 2, 300, 300, 2, 128)
    scale = 1 / math.sqrt(128)
    o, lse = lib.fwd(to_dev(q), to_dev(k), to_dev(v), scale, True)
    got = _run_bwd(lib, q, k, v, do, scale, True, o=o, lse=lse)
    torch.cuda.synchronize()
    _check(got, OB.backward_bshd(q, k, v, do, scale, True), "chained")


def test_bwd_empty_rows_no_queries_and_determinism(lib):
    import torch
    # causal with Sq > Sk: the first Sq - Sk rows see no key and pass no gradient
    q, k, v, do = _inputs(600, 1, 300, 100, 2, 64)
    scale = 0.125
    g1 = _run_bwd(lib, q, k, v, do, scale, True)
    g2 = _run_bwd(lib, q, k, v, do, scale, True)
    for a, b in zip(g1, g2):
        assert np.array_equal(a, b)
    assert (g1[0][:, :200] == 0).all()
    _check(g1, OB.backward_bshd(q, k, v, do, scale, True), "empty rows")
    # no queries: the key and value gradients are zero
    k2 = to_dev(k)
    z = torch.empty((1, 0, 2, 64), dtype=torch.bfloat16, device="cuda")
    dq, dk, dv = lib.bwd(z, k2, k2, z, torch.empty((1, 2, 0), dtype=torch.float32, device="cuda"), z, scale,
                         False)
    torch.cuda.synchronize()
    assert (dk.float() == 0).all() and (dv.float() == 0).all()


def test_bwd_ablation_shape_sampled_heads(lib):
    """batch 4, 16 heads, seq 8448, d128 (the forward's bench shape), GPU
    gradients of two (batch, head) pairs against the oracle."""
    import torch
    w = W.WORKLOADS["ablation"]
    qs, ks = w.shapes()
    q, k, v = W.qkv_normal(w.seed, qs, ks)
    do, _, _ = W.qkv_normal(w.seed + 1000, qs)
    tq, tk, tv, tdo = (to_dev(x) for x in (q, k, v, do))
    o, lse = lib.fwd(tq, tk, tv, w.scale, False)
    dq, dk, dv = lib.bwd(tq, tk, tv, o, lse, tdo, w.scale, False)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (3, 15)):
        ref = OB.backward_head(q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h], w.scale, False)
        got = tuple(t[b, :, h].float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv))
        _check(got, ref, f"ablation b{b} h{h}")
