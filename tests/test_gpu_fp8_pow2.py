"""GPU parity of the power-of-two form of the 8-bit path
(attn_fp8_quantize_pow2, attn_fwd_fp8_pow2) against the float64 oracle.

* Quantiser without rotation: codes and scales bit-exact, the premul product
  included (float32 on both sides; the division by a power of two is exact).
  With the rotation: within one e4m3 step, as for attn_fp8_quantize.
* The forward, fed the oracle's own codes (Q coded times the softmax scale
  times log2(e)), against float64 attention of the dequantised codes (the
  factor divided out of Q): the bounds of attn_fwd_fp8's test (the e4m3
  rounding of the probabilities and float32 accumulation remain).
* Rows whose running max moves again and again after the first tile.
* The outlier workload (batch 4, 16 heads, seq 8192, d128): RMSE <= 1.2e-2
  against float64 exact attention, below the per-tensor baseline of the same
  form, and within 10 % of the amax / 448 pipeline's RMSE."""
import math

import numpy as np
import pytest

import workloads as W
from oracle import attention as OA
from oracle import fp8 as OF
from tests.parity import sample_rows, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_attn_fwd_10_amd as A
    return A


def _dev_u8(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).cuda()


def _dev_f32(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("s", [128, 300])
@pytest.mark.parametrize("block_rows", [128, 0])
@pytest.mark.parametrize("premul", [1.0, 0.12751743074, 3.0])
def test_quantize_pow2_bitexact_without_rotation(lib, d, s, block_rows, premul):
    import torch
    x, _, _ = W.qkv_outlier(40 + d + s, (2, s, 3, d))
    codes, scales = lib.fp8_quantize_pow2(to_dev(x), block_rows, None, premul)
    torch.cuda.synchronize()
    rc, rs = OF.quantize_pow2(x, block_rows, premul)
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)


def _across_magnitudes(rng, shape):
    """N(0,1) blocks, each (batch, head, 128-row block) multiplied by its own
    power of two from 2^-140 (bf16 subnormals; quotients amax / 448 below the
    normal range) to 2^100, rounded to bf16."""
    B, S, H, D = shape
    x = rng.standard_normal(shape).astype(np.float64)
    exps = np.array([-140, -133, -128, -126, -100, -64, -61, -60, -59, -20, -1, 0, 3, 40, 100])
    for b in range(B):
        for h in range(H):
            for blk in range(0, S, 128):
                x[b, blk:blk + 128, h] *= 2.0 ** int(rng.choice(exps))
    return W.bf16_bits_to_f32(W.bf16_round(x.astype(np.float32)))


@pytest.mark.parametrize("block_rows", [128, 0])
def test_quantize_pow2_bitexact_across_magnitudes(lib, block_rows):
    import torch
    x = _across_magnitudes(np.random.default_rng(71 + block_rows), (2, 640, 4, 128))
    xd = to_dev(x)
    assert np.array_equal(xd.float().cpu().numpy(), x)   # bf16-exact inputs
    codes, scales = lib.fp8_quantize_pow2(xd, block_rows, None, 0.5)
    torch.cuda.synchronize()
    rc, rs = OF.quantize_pow2(x, block_rows, 0.5)
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_quantize_pow2_with_rotation_within_one_step(lib, d):
    import torch
    x, _, _ = W.qkv_outlier(50 + d, (2, 300, 3, d))
    signs = W.random_signs(4, d)
    pm = OF.LOG2E / math.sqrt(d)
    codes, scales = lib.fp8_quantize_pow2(to_dev(x), 128, torch.from_numpy(signs).cuda(), pm)
    torch.cuda.synchronize()
    xr = OF.rotate(x, signs).astype(np.float32)
    rc, rs = OF.quantize_pow2(xr, 128, pm)
    # (power-of-two scales: equal unless an amax sits within float32 rounding
    # of 448 times a power of two, which these inputs do not)
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)
    got = OF.dequantize(codes.cpu().numpy(), rs, 128)
    want = OF.dequantize(rc, rs, 128)
    sc = np.transpose(rs, (0, 2, 1))[:, np.arange(300) // 128][..., None]
    step = OF.e4m3_ulp(np.maximum(np.abs(got), np.abs(want)) / sc) * sc
    assert (np.abs(got - want) <= step * (1 + 1e-6)).all()
    assert (codes.cpu().numpy() != rc).mean() < 1e-2


def _run(lib, qp, causal):
    import torch
    o, lse = lib.fwd_fp8_pow2(_dev_u8(qp["q8"]), _dev_f32(qp["q_scale"]), _dev_u8(qp["k8"]), _dev_f32(qp["k_scale"]),
                              _dev_u8(qp["v8"]), _dev_f32(qp["v_scale"]), qp["block_rows"], causal)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _check_vs_dequantised(o, lse, qp, causal, scale):
    qd, kd, vd = OF.dequantize_pipeline(qp)
    o_ref, lse_ref = OA.attention_bshd(qd, kd, vd, scale, causal)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.abs(lse[fin] - lse_ref[fin]).max() <= 1e-3
    err = o - o_ref
    rmse = float(np.sqrt(np.mean(err ** 2)))
    assert rmse <= 5e-3, rmse
    assert np.abs(err).max() <= 6e-2, np.abs(err).max()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("block_rows", [128, 0])
@pytest.mark.parametrize("sq,sk", [(256, 256), (200, 333), (333, 200), (1, 1), (130, 64), (300, 192),
                                   (260, 1000), (700, 520)])
def test_fwd_fp8_pow2_vs_dequantised_attention(lib, causal, block_rows, sq, sk):
    d = 128
    q, k, v = W.qkv_normal(60 + sq, (2, sq, 2, d), (2, sk, 2, d))
    qp = OF.quantize_pipeline_pow2(q, k, v, W.random_signs(4, d), block_rows, scale=1 / math.sqrt(d))
    o, lse = _run(lib, qp, causal)
    _check_vs_dequantised(o, lse, qp, causal, 1 / math.sqrt(d))


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_fp8_pow2_max_moves_late(lib, causal):
    """Rows whose largest scores come in late tiles, far above the first
    tile's: the running max then moves by more than its lag after the first
    tile, again and again (the accumulators and row sums rescaled, the score
    MFMAs' starting value moved).  Key 64 t + i of tile t >= 1 gets 0.3 t
    times query i added (i < 64), so query i's best score grows by about
    0.3 * 128 / sqrt(128) * log2(e) = 4.9 base-2 units per tile, above the
    lag of 2; the block scales of K then differ from block to block too."""
    d, sq, sk = 128, 200, 700
    rng = np.random.default_rng(91)
    q = rng.standard_normal((1, sq, 2, d)).astype(np.float32)
    k = rng.standard_normal((1, sk, 2, d)).astype(np.float32)
    v = rng.standard_normal((1, sk, 2, d)).astype(np.float32)
    for t in range(1, (sk + 63) // 64):
        n = min(64, sk - 64 * t)
        k[:, 64 * t:64 * t + n] += 0.3 * t * q[:, :n]
    q, k, v = (W.bf16_bits_to_f32(W.bf16_round(x)) for x in (q, k, v))
    qp = OF.quantize_pipeline_pow2(q, k, v, None, 128, scale=1 / math.sqrt(d))
    assert len(np.unique(qp["k_scale"])) > 1
    o, lse = _run(lib, qp, causal)
    _check_vs_dequantised(o, lse, qp, causal, 1 / math.sqrt(d))


def test_fwd_fp8_pow2_empty_rows_and_determinism(lib):
    d = 128
    q, k, v = W.qkv_normal(77, (1, 300, 2, d), (1, 100, 2, d))
    qp = OF.quantize_pipeline_pow2(q, k, v, None, 128, scale=1 / math.sqrt(d))
    o1, l1 = _run(lib, qp, True)
    o2, l2 = _run(lib, qp, True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert np.all(o1[:, :200] == 0) and np.all(np.isneginf(l1[:, :, :200]))


def _rows_ref(q, k, v, scale, rows):
    B, S, H, D = q.shape
    o = np.zeros((B, len(rows), H, D))
    for b in range(B):
        for h in range(H):
            oo, _ = OA.naive_head(q[b, rows, h], k[b, :, h], v[b, :, h], scale, False, rows=rows, lq=S)
            o[b, :, h] = oo
    return o


def test_outlier_workload_accuracy_pow2(lib):
    """batch 4, 16 heads, seq 8192, d128: the power-of-two form with block-128
    scales and the random-sign Hadamard rotation against its per-tensor
    baseline, and beside the amax / 448 pipeline, all through the GPU."""
    import torch
    w = W.WORKLOADS["fp8"]
    qs, _ = w.shapes()
    q, k, v = W.qkv_outlier(w.seed, qs)
    signs = torch.from_numpy(W.random_signs(4, w.head_dim)).cuda()
    tq, tk, tv = to_dev(q), to_dev(k), to_dev(v)
    rows = sample_rows(w.seq_q, seed=31, n_random=40)
    o_ref = _rows_ref(q, k, v, w.scale, rows)
    out = {}
    for name, br, sg in (("block+hadamard", 128, signs), ("per-tensor", 0, None)):
        q8, qsc = lib.fp8_quantize_pow2_q(tq, w.scale, br, sg)
        k8, ksc = lib.fp8_quantize_pow2(tk, br, sg)
        v8, vsc = lib.fp8_quantize_pow2(tv, br, None)
        o, _ = lib.fwd_fp8_pow2(q8, qsc, k8, ksc, v8, vsc, br, False)
        torch.cuda.synchronize()
        out[name] = OF.rmse(o[:, rows].float().cpu().numpy().astype(np.float64), o_ref)
    q8, qsc = lib.fp8_quantize(tq, 128, signs)
    k8, ksc = lib.fp8_quantize(tk, 128, signs)
    v8, vsc = lib.fp8_quantize(tv, 128, None)
    o, _ = lib.fwd_fp8(q8, qsc, k8, ksc, v8, vsc, 128, w.scale, False)
    torch.cuda.synchronize()
    out["amax/448 block+hadamard"] = OF.rmse(o[:, rows].float().cpu().numpy().astype(np.float64), o_ref)
    print(out)
    assert out["block+hadamard"] <= 1.2e-2, out
    assert out["block+hadamard"] < out["per-tensor"], out
    assert out["block+hadamard"] <= 1.1 * out["amax/448 block+hadamard"], out
