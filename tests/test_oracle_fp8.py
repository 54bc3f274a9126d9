"""Pins for the 8-bit oracle pieces (CPU only): the e4m3 codec against the format
definition (tests/golden) and torch's float8_e4m3fn, the Hadamard rotation
against scipy and the orthogonality identities, and the quantisers against
their defining properties."""
import json
import math
import os

import numpy as np
import pytest

from oracle import attention as A
from oracle import fp8 as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_decode_golden_points():
    with open(os.path.join(GOLDEN, "e4m3fn_points.json")) as f:
        g = json.load(f)
    for p in g["points"]:
        assert F.e4m3_decode(np.uint8(p["code"])) == p["value"], p
    for c in g["nan_codes"]:
        assert np.isnan(F.e4m3_decode(np.uint8(c)))
    for r in g["rounding"]:
        assert int(F.e4m3_encode(np.float64(r["x"]))) == r["code"], r


def test_decode_exhaustive_vs_torch():
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    ours = F.e4m3_decode(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ours)
    assert np.array_equal(ours[fin], ref[fin])


def test_encode_roundtrip_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    vals = F.e4m3_decode(codes)
    fin = ~np.isnan(vals)
    back = F.e4m3_encode(vals[fin])
    assert np.array_equal(back, codes[fin])
    assert (F.e4m3_encode(np.array([np.nan])) == F.E4M3_NAN).all()


def test_encode_vs_torch_random():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    # values across the whole range incl. subnormals, in float32 like the kernel
    x = (rng.standard_normal(200000) * np.exp2(rng.uniform(-12, 8.7, 200000))).astype(np.float32)
    x = x[np.abs(x) <= 448]
    ours = F.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_encode_ties_to_even_between_every_pair():
    codes = np.arange(0, 126, dtype=np.uint8)          # positive finite codes 0..125
    lo = F.e4m3_decode(codes)
    hi = F.e4m3_decode(codes + 1)
    mid = (lo + hi) / 2
    got = F.e4m3_encode(mid)
    want = np.where(codes % 2 == 0, codes, codes + 1)
    assert np.array_equal(got, want)


def test_saturation():
    assert int(F.e4m3_encode(np.float64(1e30))) == 0x7E
    assert int(F.e4m3_encode(np.float64(-465.0))) == 0xFE
    assert int(F.e4m3_encode(np.float64(447.9))) == 0x7E


def test_hadamard_orthogonality_and_scipy():
    scipy_linalg = pytest.importorskip("scipy.linalg")
    for d in (1, 2, 8, 64, 128, 256):
        h = F.sylvester_hadamard(d)
        assert np.array_equal(h @ h.T, d * np.eye(d, dtype=np.int64))
        assert np.array_equal(h, scipy_linalg.hadamard(d))


@pytest.mark.parametrize("d", [64, 128, 256])
def test_fwht_equals_dense_product(d):
    rng = np.random.default_rng(d)
    x = rng.standard_normal((5, 3, d))
    np.testing.assert_allclose(F.fwht(x), x @ F.sylvester_hadamard(d), rtol=0, atol=1e-11)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_rotation_cancels_in_qk(d):
    rng = np.random.default_rng(d + 1)
    signs = np.where(rng.random(d) < 0.5, -1, 1)
    m = F.rotation_matrix(signs)
    np.testing.assert_allclose(m @ m.T, np.eye(d), rtol=0, atol=1e-13)
    q, k = rng.standard_normal((20, d)), rng.standard_normal((30, d))
    qr, kr = F.rotate(q, signs), F.rotate(k, signs)
    np.testing.assert_allclose(qr @ kr.T, q @ k.T, rtol=0, atol=1e-12)
    np.testing.assert_allclose(qr, q @ m, rtol=0, atol=1e-12)
    # and so attention is unchanged by the rotation
    v = rng.standard_normal((30, d))
    o1, l1 = A.naive_head(q, k, v, 0.1)
    o2, l2 = A.naive_head(qr, kr, v, 0.1)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-12)


def test_block_quantiser_properties():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 300, 3, 64)).astype(np.float32)
    x[1, 130:256, 2] = 0.0                              # an all-zero block -> scale 1
    codes, scales = F.quantize(x, 128)
    assert scales.shape == (2, 3, 3)
    for b in range(2):
        for h in range(3):
            for i in range(3):
                blk = x[b, i * 128:(i + 1) * 128, h]
                amax = np.abs(blk).max()
                if amax == 0:
                    assert scales[b, h, i] == 1.0
                    assert (codes[b, i * 128:(i + 1) * 128, h] == 0).all()
                    continue
                assert scales[b, h, i] == np.float32(amax) / np.float32(448)
                c = codes[b, i * 128:(i + 1) * 128, h]
                # the largest magnitude lands on (or rounds to) the top code
                assert ((c & 0x7F) == 0x7E).any()
    deq = F.dequantize(codes, scales, 128)
    # error at most half an e4m3 spacing (in scaled units) plus float32 division rounding
    sc = np.transpose(scales, (0, 2, 1))[:, np.arange(300) // 128][..., None]
    err = np.abs(deq - x) / sc
    assert (err <= 0.5 * F.e4m3_ulp(x / sc) * (1 + 1e-6) + 1e-30).all()


def test_per_tensor_quantiser():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((1, 50, 2, 64)).astype(np.float32)
    codes, scales = F.quantize(x, 0)
    assert scales.shape == (1,)
    assert scales[0] == np.float32(np.abs(x).max()) / np.float32(448)
    deq = F.dequantize(codes, scales, 0)
    np.testing.assert_allclose(deq, x, rtol=0.0625, atol=2.0 ** -9 * scales[0])


def test_emulation_prediction_block_rotation_beats_per_tensor():
    """The page's accuracy claim on a small outlier workload: block
    quantisation with rotation has lower RMSE than per-tensor scaling."""
    import workloads as W
    B, S, H, D = 1, 512, 2, 128
    q, k, v = W.qkv_outlier(11, (B, S, H, D))
    signs = W.random_signs(4, D)
    sc = 1 / math.sqrt(D)
    ref, _ = A.attention_bshd(q, k, v, sc)
    blk, _ = F.emulate_fp8_attention(q, k, v, sc, signs=signs, block_rows=128)
    pt, _ = F.emulate_fp8_attention(q, k, v, sc, signs=None, block_rows=0)
    r_blk, r_pt = F.rmse(blk, ref), F.rmse(pt, ref)
    assert r_blk < r_pt
    assert r_blk < 1.2e-2


def test_rmse_golden():
    """The pass measure of the 8-bit configs, against hand-derived values."""
    with open(os.path.join(GOLDEN, "oracle_measures.json")) as f:
        g = json.load(f)
    for c in g["rmse"]:
        assert F.rmse(np.array(c["a"], float), np.array(c["b"], float)) == pytest.approx(c["value"], abs=1e-15), c
        assert F.rmse(np.array(c["b"], float), np.array(c["a"], float)) == pytest.approx(c["value"], abs=1e-15), c


def test_e4m3_ulp_golden():
    with open(os.path.join(GOLDEN, "oracle_measures.json")) as f:
        g = json.load(f)
    for c in g["e4m3_ulp"]:
        assert float(F.e4m3_ulp(np.float64(c["x"]))) == c["value"], c


def test_e4m3_ulp_is_the_spacing_of_adjacent_codes():
    """For every non-negative finite code but the largest, the step to the next
    code (decoded by the codec pinned above) is e4m3_ulp of the code's value."""
    codes = np.arange(0, 126, dtype=np.uint8)
    lo = F.e4m3_decode(codes)
    hi = F.e4m3_decode(codes + 1)
    assert np.array_equal(hi - lo, F.e4m3_ulp(lo))
    assert np.array_equal(F.e4m3_ulp(-lo), F.e4m3_ulp(lo))


@pytest.mark.parametrize("fmt", ["bf16", "fp16"])
def test_half_ulp_of_16bit_outputs(fmt):
    """The rounding allowance of the 16-bit parity tests: twice half_ulp(x) is
    the step from x to the next representable value, for values across the
    normal range of each format (bit patterns stepped by one)."""
    from tests.parity import half_ulp
    rng = np.random.default_rng(3)
    if fmt == "bf16":
        bits = rng.integers(0x0080, 0x7F7F, size=5000).astype(np.uint32)
        x = (bits << 16).view(np.float32).astype(np.float64)
        nxt = ((bits + 1) << 16).view(np.float32).astype(np.float64)
    else:
        bits = rng.integers(0x0400, 0x7BFF, size=5000).astype(np.uint16)
        x = bits.view(np.float16).astype(np.float64)
        nxt = (bits + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    assert np.array_equal(2 * half_ulp(x, fmt), nxt - x)
    assert half_ulp(1.0, fmt) == (2.0 ** -8 if fmt == "bf16" else 2.0 ** -11)


# ---------------------------------------------------------------------------
# the power-of-two form
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("amax,scale", [
    (448.0, 1.0),                  # amax / 448 = 1 exactly
    (447.99, 1.0),
    (449.0, 2.0),                  # just above a power of two: the next one
    (672.0, 2.0),                  # 1.5
    (224.0, 0.5),
    (223.9, 0.5),
    (448.0 * 2.0 ** -20, 2.0 ** -20),
    (3.0e38, 2.0 ** 120),          # 6.7e35 lies in (2^119, 2^120]
    (1e-40, 2.0 ** -126),          # quotient below the normal range: the floor
    (2.0 ** -149, 2.0 ** -126),    # quotient that rounds to zero
    (0.0, 1.0),                    # an all-zero block
])
def test_pow2_scale_values(amax, scale):
    """Hand-derived values of the power-of-two scale rule (smallest power of
    two at or above float32(amax / 448), at least 2^-126, 1 for amax = 0)."""
    assert float(F.scale_pow2_from_amax(np.float32(amax))) == scale


def test_pow2_block_quantiser_properties():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 300, 3, 64)).astype(np.float32)
    x[1, 130:256, 2] = 0.0                              # an all-zero block -> scale 1
    codes, scales = F.quantize_pow2(x, 128)
    assert scales.shape == (2, 3, 3)
    for b in range(2):
        for h in range(3):
            for i in range(3):
                blk = x[b, i * 128:(i + 1) * 128, h]
                amax = np.abs(blk).max()
                if amax == 0:
                    assert scales[b, h, i] == 1.0
                    assert (codes[b, i * 128:(i + 1) * 128, h] == 0).all()
                    continue
                sc = float(scales[b, h, i])
                t = float(np.float32(amax) / np.float32(448))
                # a power of two, the smallest at or above amax / 448
                assert np.frexp(sc)[0] == 0.5
                assert sc >= t and sc / 2 < t
                # so the largest magnitude, in (224, 448] after the division,
                # codes to a value in [224, 448]
                top = np.abs(F.e4m3_decode(codes[b, i * 128:(i + 1) * 128, h])).max()
                assert 224 <= top <= 448
    deq = F.dequantize(codes, scales, 128)
    # error at most half an e4m3 spacing (in scaled units): the division is exact
    sc = np.transpose(scales, (0, 2, 1))[:, np.arange(300) // 128][..., None]
    err = np.abs(deq - x) / sc
    assert (err <= 0.5 * F.e4m3_ulp(x / sc)).all()
    # per tensor: the same rule over the whole tensor
    c0, s0 = F.quantize_pow2(x, 0)
    t = float(np.float32(np.abs(x).max()) / np.float32(448))
    assert s0.shape == (1,) and np.frexp(float(s0[0]))[0] == 0.5 and s0[0] >= t and s0[0] / 2 < t


def test_pow2_premul_invariance_and_error():
    """Multiplying by a power of two moves the scales by it and leaves the codes
    alone (every step of the rule is exact under it); any premul codes
    x * premul to within half an e4m3 step in scaled units."""
    rng = np.random.default_rng(9)
    x = rng.standard_normal((1, 260, 2, 64)).astype(np.float32)
    c0, s0 = F.quantize_pow2(x, 128)
    for k in (-7, 3):
        c1, s1 = F.quantize_pow2(x, 128, premul=2.0 ** k)
        assert np.array_equal(c1, c0)
        assert np.array_equal(s1, s0 * np.float32(2.0 ** k))
    pm = 0.0883883476 * 1.4426950408889634
    c2, s2 = F.quantize_pow2(x, 128, premul=pm)
    xp = (x * np.float32(pm)).astype(np.float64)
    sc = np.transpose(s2, (0, 2, 1))[:, np.arange(260) // 128][..., None].astype(np.float64)
    err = np.abs(F.dequantize(c2, s2, 128) - xp) / sc
    assert (err <= 0.5 * F.e4m3_ulp(xp / sc)).all()


def test_pow2_pipeline_premul_cancels():
    """quantize_pipeline_pow2 codes Q times the softmax scale times log2(e);
    dequantize_pipeline divides that factor out again, so the dequantised Q'
    is Q' to within the e4m3 rounding, and the emulated attention is close to
    that of the amax / 448 pipeline."""
    rng = np.random.default_rng(10)
    q, k, v = (rng.standard_normal((1, 130, 2, 128)).astype(np.float32) for _ in range(3))
    sc = 1 / math.sqrt(128)
    qp = F.quantize_pipeline_pow2(q, k, v, None, 128, scale=sc)
    assert qp["q_premul"] == pytest.approx(1.4426950408889634 * sc, rel=1e-15)
    qd, kd, vd = F.dequantize_pipeline(qp)
    assert np.abs(qd - q).max() <= np.abs(q).max() * 2.0 ** -4
    ref, _ = A.attention_bshd(q, k, v, sc)
    o2, _ = A.attention_bshd(qd, kd, vd, sc)
    o1, _ = A.attention_bshd(*F.dequantize_pipeline(F.quantize_pipeline(q, k, v, None, 128)), sc)
    assert F.rmse(o2, ref) < 2 * F.rmse(o1, ref)
