"""Pins for the int8 oracle pieces (CPU only): the symmetric int8 code against
its definition (hand-worked points, every code, torch's rounding), the block
and per-tensor quantisers against their defining properties, and the accuracy
ordering of block quantisation with rotation against per-tensor scaling."""
import math

import numpy as np
import pytest

from oracle import attention as A
from oracle import int8 as I


def test_encode_worked_points():
    """Scaled values and the codes the reading fixes for them (nearest, ties to
    even, clamp to +-127), worked by hand."""
    pts = [(63.5, 64), (62.5, 62), (0.5, 0), (-0.5, 0), (1.5, 2), (-1.5, -2), (2.4999, 2),
           (126.6, 127), (127.4, 127), (300.0, 127), (-300.0, -127), (-126.5, -126), (0.0, 0)]
    for y, c in pts:
        assert int(I.int8_encode(np.float32(y))) == c, (y, c)


def test_every_code_round_trips_and_rounds_to_itself():
    c = np.arange(-127, 128)
    assert (I.int8_encode(I.int8_decode(c).astype(np.float32)) == c).all()
    assert (I.int8_encode((c + 0.49).astype(np.float32))[:-1] == c[:-1]).all()
    assert (I.int8_encode((c - 0.49).astype(np.float32))[1:] == c[1:]).all()
    assert I.int8_encode(np.float32(-128.0)) == -127  # -128 is never produced


def test_encode_vs_torch_rounding():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    y = (rng.standard_normal(20000) * 60).astype(np.float32)
    y[:200] = np.round(y[:200]) + 0.5          # exact ties
    ref = torch.clamp(torch.round(torch.from_numpy(y)), -127, 127).to(torch.int8).numpy()
    assert (I.int8_encode(y) == ref).all()


def test_block_quantiser_properties():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 300, 3, 64)).astype(np.float32)
    x[1, 130:256, 2] = 0.0                                 # an all-zero block -> scale 1
    codes, scales = I.quantize(x, 128)
    assert codes.dtype == np.int8 and scales.shape == (2, 3, 3)
    for b in range(2):
        for h in range(3):
            for i in range(3):
                blk = x[b, i * 128:(i + 1) * 128, h]
                c = codes[b, i * 128:(i + 1) * 128, h]
                amax = np.abs(blk).max()
                if amax == 0:
                    assert scales[b, h, i] == 1.0 and (c == 0).all()
                    continue
                assert scales[b, h, i] == np.float32(amax) / np.float32(127)
                assert np.abs(c.astype(np.int32)).max() == 127   # the amax element takes the top code
    deq = I.dequantize(codes, scales, 128)
    sc = np.transpose(scales, (0, 2, 1))[:, np.arange(300) // 128][..., None]
    assert (np.abs(deq - x) <= 0.5 * sc * (1 + 1e-5)).all()


def test_per_tensor_quantiser():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((1, 50, 2, 64)).astype(np.float32)
    codes, scales = I.quantize(x, 0)
    assert scales.shape == (1,) and scales[0] == np.float32(np.abs(x).max()) / np.float32(127)
    deq = I.dequantize(codes, scales, 0)
    assert np.abs(deq - x).max() <= 0.5 * scales[0] * (1 + 1e-5)


def test_emulation_block_rotation_beats_per_tensor():
    """On the outlier workload shape, block scales with the rotation give a
    lower attention RMSE than one scale per tensor."""
    import workloads as W
    B, S, H, D = 1, 512, 2, 128
    q, k, v = W.qkv_outlier(11, (B, S, H, D))
    signs = W.random_signs(4, D)
    sc = 1 / math.sqrt(D)
    ref, _ = A.attention_bshd(q, k, v, sc)
    blk, _ = I.emulate_int8_attention(q, k, v, sc, signs=signs, block_rows=128)
    pt, _ = I.emulate_int8_attention(q, k, v, sc, signs=None, block_rows=0)
    r_blk = float(np.sqrt(np.mean((blk - ref) ** 2)))
    r_pt = float(np.sqrt(np.mean((pt - ref) ** 2)))
    print(f"int8 emulation rmse: block+rotation {r_blk:.3e}, per-tensor {r_pt:.3e}")
    assert r_blk < r_pt
    assert r_blk < 1.2e-2


def test_pipeline_formats():
    """Q and K become int8 codes with int8 scales (amax/127), V keeps the e4m3
    codes and scales of the 8-bit path."""
    from oracle import fp8 as F
    rng = np.random.default_rng(9)
    x = rng.standard_normal((1, 200, 2, 128)).astype(np.float32)
    qp = I.quantize_pipeline(x, x, x, None, 128)
    assert qp["q8"].dtype == np.int8 and qp["k8"].dtype == np.int8
    assert (qp["q8"] == I.quantize(x, 128)[0]).all()
    v8, vs = F.quantize(x, 128)
    assert (qp["v8"] == v8).all() and (qp["v_scale"] == vs).all()
    qd, kd, vd = I.dequantize_pipeline(qp)
    assert np.abs(qd - x).max() <= 0.5 * qp["q_scale"].max() * (1 + 1e-5)
    assert np.abs(vd - x).max() <= 0.5 * F.e4m3_ulp(np.abs(x) / vs.min()).max() * vs.max()


def test_reading_fixed_point_probabilities_are_too_coarse():
    """Why the output product keeps e4m3 probabilities: with the same
    dequantised inputs, probabilities rounded to int8 fixed point (127 = the
    row maximum) give a far larger attention error on the outlier workload
    than probabilities rounded to e4m3 (p * 2^6, as the 8-bit path does)."""
    import workloads as W
    from oracle import fp8 as F
    B, S, H, D = 1, 2048, 1, 128
    q, k, v = W.qkv_outlier(21, (B, S, H, D))
    signs = W.random_signs(4, D)
    sc = 1 / math.sqrt(D)
    rows = np.arange(0, S, 16)
    ref = A.attention_bshd(q, k, v, sc, rows=rows)[0][0, rows, 0]
    qd, kd, vd = I.dequantize_pipeline(I.quantize_pipeline(q, k, v, signs, 128))
    s = qd[0, rows, 0] @ kd[0, :, 0].T * sc
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p_fixed = np.rint(p * 127)
    p_e4m3 = F.e4m3_decode(F.e4m3_encode((p * 64).astype(np.float32)))
    err = {}
    for name, pp in (("fixed", p_fixed), ("e4m3", p_e4m3)):
        o = (pp @ vd[0, :, 0]) / pp.sum(axis=1, keepdims=True)
        err[name] = float(np.sqrt(np.mean((o - ref) ** 2)))
    print(f"rmse: int8 fixed-point P {err['fixed']:.3e}, e4m3 P {err['e4m3']:.3e}")
    assert err["fixed"] > 4 * err["e4m3"]
    assert err["e4m3"] < 1.2e-2
