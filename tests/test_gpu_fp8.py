"""GPU parity of the 8-bit path: the quantisation prologue (attn_fp8_quantize)
and the e4m3 forward (attn_fwd_fp8), against the float64 oracle.

* Quantiser without rotation: codes and scales are bit-exact (the code decision
  is taken in float32 on both sides).  With the rotation the GPU evaluates the
  Hadamard transform in float32 and the oracle in float64, so codes may differ
  by one e4m3 step where the rotated value sits on a rounding boundary.
* The e4m3 forward, fed the oracle's own codes, is compared with float64
  attention of the dequantised codes; the remaining difference is the e4m3
  rounding of the probabilities (relative error <= 2^-4 per probability,
  averaged over many keys) and float32 accumulation.
* On the outlier workload (batch 4, 16 heads, seq 8192, d128, 0.1 % N(0,100)
  outliers) the full pipeline must reach RMSE <= 1.2e-2 against float64 exact
  attention and beat the per-tensor-scaled baseline built in the same run."""
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
def test_quantize_bitexact_without_rotation(lib, d, s, block_rows):
    import torch
    x, _, _ = W.qkv_outlier(40 + d + s, (2, s, 3, d))
    codes, scales = lib.fp8_quantize(to_dev(x), block_rows, None)
    torch.cuda.synchronize()
    rc, rs = OF.quantize(x, block_rows)
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)


def _e4m3_boundary_values(rng, shape):
    """Values whose quotient by the scale falls on every e4m3 code, on every
    rounding tie between neighbouring codes (normal and subnormal), one bf16
    step either side of each tie, and below half the smallest subnormal (which
    must give a signed zero), in both signs.  Every (batch, head, 128-row block)
    holds +-28, so its scale is 28 / 448 = 2^-4 and the division is exact."""
    vals = OF.e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    step = 2.0 ** (np.floor(np.log2(np.abs(mids))) - 7)     # one bf16 step
    y = np.concatenate([vals, mids, mids + step, mids - step, [2.0 ** -11, 2.0 ** -13]])
    y = np.concatenate([y, -y]) / 16.0
    x = rng.permutation(np.resize(y, int(np.prod(shape)))).reshape(shape)
    x[:, ::128, :, 0] = 28.0
    x[:, 1::128, :, 1] = -28.0
    return x


@pytest.mark.parametrize("block_rows", [128, 0])
def test_quantize_rounding_ties_bitexact(lib, block_rows):
    import torch
    x = _e4m3_boundary_values(np.random.default_rng(7), (2, 300, 2, 64))
    assert np.array_equal(to_dev(x).float().cpu().numpy(), x)   # bf16-exact inputs
    codes, scales = lib.fp8_quantize(to_dev(x), block_rows, None)
    torch.cuda.synchronize()
    rc, rs = OF.quantize(x, block_rows)
    assert np.all(rs == np.float32(2.0 ** -4))
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)


def _across_magnitudes(rng, shape):
    """N(0,1) blocks, each (batch, head, 128-row block) multiplied by its own
    power of two from 2^-140 (bf16 subnormals, and a scale below 2^-60 whose
    reciprocal would overflow) to 2^100, rounded to bf16."""
    B, S, H, D = shape
    x = rng.standard_normal(shape).astype(np.float64)
    exps = np.array([-140, -133, -128, -126, -100, -64, -61, -60, -59, -20, -1, 0, 3, 40, 100])
    for b in range(B):
        for h in range(H):
            for blk in range(0, S, 128):
                x[b, blk:blk + 128, h] *= 2.0 ** int(rng.choice(exps))
    bits = W.bf16_round(x.astype(np.float32))
    return W.bf16_bits_to_f32(bits)


@pytest.mark.parametrize("fmt", ["e4m3", "int8"])
@pytest.mark.parametrize("block_rows", [128, 0])
def test_quantize_bitexact_across_magnitudes(lib, fmt, block_rows):
    """The code decision (a correctly rounded float32 quotient x / scale, then
    the format's rounding) matches the oracle bit for bit for blocks of every
    magnitude, subnormal inputs and scales included."""
    import torch
    from oracle import int8 as OI
    x = _across_magnitudes(np.random.default_rng(61 + block_rows), (2, 640, 4, 128))
    xd = to_dev(x)
    assert np.array_equal(xd.float().cpu().numpy(), x)   # bf16-exact inputs
    if fmt == "e4m3":
        codes, scales = lib.fp8_quantize(xd, block_rows, None)
        rc, rs = OF.quantize(x, block_rows)
    else:
        codes, scales = lib.int8_quantize(xd, block_rows, None)
        rc, rs = OI.quantize(x, block_rows)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_quantize_with_rotation_within_one_step(lib, d):
    import torch
    x, _, _ = W.qkv_outlier(50 + d, (2, 300, 3, d))
    signs = W.random_signs(4, d)
    codes, scales = lib.fp8_quantize(to_dev(x), 128, torch.from_numpy(signs).cuda())
    torch.cuda.synchronize()
    xr = OF.rotate(x, signs).astype(np.float32)
    rc, rs = OF.quantize(xr, 128)
    np.testing.assert_allclose(scales.cpu().numpy(), rs, rtol=1e-5, atol=0)
    got = OF.dequantize(codes.cpu().numpy(), rs, 128)
    want = OF.dequantize(rc, rs, 128)
    # at most one e4m3 step (in scaled units) apart, and nearly always equal
    sc = np.transpose(rs, (0, 2, 1))[:, np.arange(300) // 128][..., None]
    step = OF.e4m3_ulp(np.maximum(np.abs(got), np.abs(want)) / sc) * sc
    assert (np.abs(got - want) <= step * (1 + 1e-6)).all()
    assert (codes.cpu().numpy() != rc).mean() < 1e-2


def _fp8_inputs_from_oracle(q, k, v, signs, block_rows):
    qp = OF.quantize_pipeline(q, k, v, signs, block_rows)
    return qp


def _run_fp8(lib, qp, causal, scale):
    import torch
    o, lse = lib.fwd_fp8(_dev_u8(qp["q8"]), _dev_f32(qp["q_scale"]), _dev_u8(qp["k8"]), _dev_f32(qp["k_scale"]),
                         _dev_u8(qp["v8"]), _dev_f32(qp["v_scale"]), qp["block_rows"], scale, causal)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("block_rows", [128, 0])
@pytest.mark.parametrize("sq,sk", [(256, 256), (200, 333), (333, 200), (1, 1), (130, 64), (300, 192),
                                   (260, 1000), (700, 520)])
def test_fwd_fp8_vs_dequantised_attention(lib, causal, block_rows, sq, sk):
    d = 128
    q, k, v = W.qkv_normal(60 + sq, (2, sq, 2, d), (2, sk, 2, d))
    signs = W.random_signs(4, d)
    qp = _fp8_inputs_from_oracle(q, k, v, signs, block_rows)
    o, lse = _run_fp8(lib, qp, causal, 1 / math.sqrt(d))
    qd = OF.dequantize(qp["q8"], qp["q_scale"], block_rows)
    kd = OF.dequantize(qp["k8"], qp["k_scale"], block_rows)
    vd = OF.dequantize(qp["v8"], qp["v_scale"], block_rows)
    o_ref, lse_ref = OA.attention_bshd(qd, kd, vd, 1 / math.sqrt(d), causal)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.abs(lse[fin] - lse_ref[fin]).max() <= 1e-3
    err = o - o_ref
    rmse = float(np.sqrt(np.mean(err ** 2)))
    assert rmse <= 5e-3, rmse
    assert np.abs(err).max() <= 6e-2, np.abs(err).max()


def test_fwd_fp8_empty_rows_and_determinism(lib):
    import torch
    d = 128
    q, k, v = W.qkv_normal(77, (1, 300, 2, d), (1, 100, 2, d))
    qp = _fp8_inputs_from_oracle(q, k, v, None, 128)
    o1, l1 = _run_fp8(lib, qp, True, 1 / math.sqrt(d))
    o2, l2 = _run_fp8(lib, qp, True, 1 / math.sqrt(d))
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


def test_outlier_workload_accuracy(lib):
    """batch 4, 16 heads, seq 8192, d128: block-128 scales + random-sign
    Hadamard vs per-tensor scales, both through the GPU pipeline."""
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
        q8, qsc = lib.fp8_quantize(tq, br, sg)
        k8, ksc = lib.fp8_quantize(tk, br, sg)
        v8, vsc = lib.fp8_quantize(tv, br, None)
        o, _ = lib.fwd_fp8(q8, qsc, k8, ksc, v8, vsc, br, w.scale, False)
        torch.cuda.synchronize()
        o = o[:, rows].float().cpu().numpy().astype(np.float64)
        out[name] = OF.rmse(o, o_ref)
    print(out)
    assert out["block+hadamard"] <= 1.2e-2, out
    assert out["block+hadamard"] < out["per-tensor"], out
