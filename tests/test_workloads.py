"""The seeded generators: bf16 rounding against torch's cast, determinism and
the structure of the varlen / paged inputs (CPU only)."""
import numpy as np
import pytest

import workloads as W


def test_bf16_round_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp2(rng.uniform(-30, 30, 100000))).astype(np.float32)
    ours = W.bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(W.bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generators_are_seeded():
    a = W.qkv_normal(5, (1, 8, 2, 4))
    b = W.qkv_normal(5, (1, 8, 2, 4))
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    assert not np.array_equal(a[0], a[1])


def test_outlier_rate():
    q, _, _ = W.qkv_outlier(3, (1, 2048, 4, 128))
    frac = (np.abs(q) > 6).mean()
    assert 2e-4 < frac < 2e-3


def test_paged_layout_is_a_permutation():
    lens = W.varlen_lengths(5, 32, 128, 4096)
    assert lens.min() >= 128 and lens.max() <= 4096
    table, total = W.paged_layout(6, lens, 64)
    used = np.concatenate([table[b, :(n + 63) // 64] for b, n in enumerate(lens)])
    assert np.array_equal(np.sort(used), np.arange(total))
    assert (table[table >= 0] < total).all()
