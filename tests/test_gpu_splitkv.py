"""GPU tests of the split-key forward (attn_fwd_splitkv): short query blocks
over long, optionally paged key caches, with the keys of every sequence cut
into ranges that run as separate work items and are merged through their
logsumexps.  The result is checked against the float64 oracle's attention over
all keys (splitting is exact up to rounding), for every row and head."""
import math

import numpy as np
import pytest

import workloads as W
from oracle import attention as OA
from tests.parity import assert_close16, to_dev, to_host
from tests.test_gpu_varlen import _pack, _paginate, _t32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_attn_fwd_10_amd as A
    return A


def _run(lib, q, k, v, cu_q, cu_k, lens_q, lens_k, causal, splits, table=None, page=0, dtype="bf16"):
    import torch
    tq, tk, tv = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    o, lse = lib.fwd_splitkv(tq, _t32(cu_q), tk, tv, _t32(cu_k), int(max(lens_q)), int(max(lens_k)),
                             causal=causal, block_table=None if table is None else _t32(table), page_size=page,
                             num_splits=splits)
    torch.cuda.synchronize()
    return to_host(o), lse.cpu().numpy().astype(np.float64)


def _reference(q, k, v, cu_q, cu_k, lens_q, lens_k, causal):
    o, lse = OA.attention_varlen(q, cu_q, k, v, cu_k, 1 / math.sqrt(q.shape[2]), causal)
    return o, lse


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("splits", [1, 2, 7, 64])
def test_decode_packed(lib, d, causal, splits):
    # one to three query rows per sequence over 63 .. 4097 keys; 64 splits leave
    # most ranges of the short sequences empty
    lens_q, lens_k = [1, 3, 1], [1000, 63, 4097]
    q, k, v, cu_q, cu_k = _pack(lens_q, lens_k, 4, d, seed=900 + d)
    o, lse = _run(lib, q, k, v, cu_q, cu_k, lens_q, lens_k, causal, splits)
    o_ref, lse_ref = _reference(q, k, v, cu_q, cu_k, lens_q, lens_k, causal)
    assert_close16(o, o_ref, lse, lse_ref, f"decode d{d} causal={causal} splits={splits}")


@pytest.mark.parametrize("causal", [False, True])
def test_decode_paged_poisoned(lib, causal):
    # paged cache of 64-token pages at shuffled physical slots, NaN in every
    # slot no sequence owns
    lens_q, lens_k = [2, 1, 4, 1], [5000, 130, 64, 2500]
    q, k, v, cu_q, cu_k = _pack(lens_q, lens_k, 8, 128, seed=910)
    kp, vp, table = _paginate(k, v, cu_k, lens_k, 64, seed=911)
    o, lse = _run(lib, q, kp, vp, cu_q, cu_k, lens_q, lens_k, causal, 8, table=table, page=64)
    o_ref, lse_ref = _reference(q, k, v, cu_q, cu_k, lens_q, lens_k, causal)
    assert_close16(o, o_ref, lse, lse_ref, f"paged decode causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_prefill_blocks_times_splits(lib, causal):
    # several 128-row query blocks per sequence, each split three ways
    lens = [300, 130, 257]
    q, k, v, cu_q, cu_k = _pack(lens, lens, 2, 128, seed=920)
    o, lse = _run(lib, q, k, v, cu_q, cu_k, lens, lens, causal, 3)
    o_ref, lse_ref = _reference(q, k, v, cu_q, cu_k, lens, lens, causal)
    assert_close16(o, o_ref, lse, lse_ref, f"prefill causal={causal}")


def test_fp16_and_auto_split_count(lib):
    lens_q, lens_k = [1, 1], [3000, 20000]
    q, k, v, cu_q, cu_k = _pack(lens_q, lens_k, 2, 128, seed=930)
    q, k, v = (W.f16_round(x).astype(np.float32) for x in (q, k, v))
    o, lse = _run(lib, q, k, v, cu_q, cu_k, lens_q, lens_k, False, None, dtype="fp16")
    o_ref, lse_ref = _reference(q, k, v, cu_q, cu_k, lens_q, lens_k, False)
    assert_close16(o, o_ref, lse, lse_ref, "fp16 auto splits", dtype="fp16")


def test_matches_unsplit_kernel(lib):
    # with one split the entry point is attn_fwd_varlen itself: bit-identical
    import torch
    lens_q, lens_k = [1, 5], [700, 900]
    q, k, v, cu_q, cu_k = _pack(lens_q, lens_k, 4, 128, seed=940)
    o1, l1 = _run(lib, q, k, v, cu_q, cu_k, lens_q, lens_k, True, 1)
    tq, tk, tv = to_dev(q), to_dev(k), to_dev(v)
    o2, l2 = lib.fwd_varlen(tq, _t32(cu_q), tk, tv, _t32(cu_k), 5, 900, causal=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(o1, to_host(o2))
    np.testing.assert_array_equal(l1, l2.cpu().numpy().astype(np.float64))


# One query row per sequence with at least 512 (sequence, key range, head)
# items is the streaming decode kernel's case (packed caches and paged caches
# of any page size); fewer items take the tiled kernel.

@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("splits", [2, 7, 64])
def test_one_row_decode_packed(lib, d, dtype, causal, splits):
    # key counts: several tiles with a ragged tail, one key, none, one short of
    # a tile, exactly a tile, and a sequence without a query row; 7 x 40 heads
    lens_q, lens_k = [1, 1, 1, 1, 1, 0, 1], [1000, 1, 0, 63, 64, 50, 4097]
    q, k, v, cu_q, cu_k = _pack(lens_q, lens_k, 40, d, seed=950 + d)
    if dtype == "fp16":
        q, k, v = (W.f16_round(x).astype(np.float32) for x in (q, k, v))
    o, lse = _run(lib, q, k, v, cu_q, cu_k, lens_q, lens_k, causal, splits, dtype=dtype)
    o_ref, lse_ref = _reference(q, k, v, cu_q, cu_k, lens_q, lens_k, causal)
    assert_close16(o, o_ref, lse, lse_ref, f"one-row decode d{d} {dtype} causal={causal} splits={splits}", dtype=dtype)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("page", [64, 256, 16, 32])
def test_one_row_decode_paged_poisoned(lib, d, page):
    # pages at shuffled physical slots, NaN in every slot no sequence owns
    # (16- and 32-token pages: every row through the table)
    lens_q, lens_k = [1, 1, 1, 1], [5000, 130, 64, 2500]
    q, k, v, cu_q, cu_k = _pack(lens_q, lens_k, 16, d, seed=960 + page + d)
    kp, vp, table = _paginate(k, v, cu_k, lens_k, page, seed=961)
    o, lse = _run(lib, q, kp, vp, cu_q, cu_k, lens_q, lens_k, True, 9, table=table, page=page)
    o_ref, lse_ref = _reference(q, k, v, cu_q, cu_k, lens_q, lens_k, True)
    assert_close16(o, o_ref, lse, lse_ref, f"one-row paged decode d{d} page={page}")


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("page", [16, 32])
def test_one_row_decode_small_pages_fp16(lib, d, page):
    # fp16 through the small-page addressing, with ragged and one-key sequences
    lens_q, lens_k = [1, 1, 1, 1], [3001, 1, 47, 1500]
    q, k, v, cu_q, cu_k = _pack(lens_q, lens_k, 16, d, seed=990 + page + d)
    q, k, v = (W.f16_round(x).astype(np.float32) for x in (q, k, v))
    kp, vp, table = _paginate(k, v, cu_k, lens_k, page, seed=991)
    o, lse = _run(lib, q, kp, vp, cu_q, cu_k, lens_q, lens_k, False, 8, table=table, page=page, dtype="fp16")
    o_ref, lse_ref = _reference(q, k, v, cu_q, cu_k, lens_q, lens_k, False)
    assert_close16(o, o_ref, lse, lse_ref, f"one-row fp16 decode d{d} page={page}", dtype="fp16")


def test_one_row_decode_large_scores(lib):
    # scores far from zero: the running max moves across tiles and splits
    lens_q, lens_k = [1, 1], [3000, 777]
    q, k, v, cu_q, cu_k = _pack(lens_q, lens_k, 64, 128, seed=970)
    q = W.normal_bf16(np.random.default_rng(971), q.shape) * 8.0
    o, lse = _run(lib, q, k, v, cu_q, cu_k, lens_q, lens_k, False, 5)
    o_ref, lse_ref = _reference(q, k, v, cu_q, cu_k, lens_q, lens_k, False)
    assert_close16(o, o_ref, lse, lse_ref, "one-row decode, large scores")


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("page", [0, 128, 16])
def test_one_row_whole_sequence(lib, d, page):
    # one key range (attn_fwd_varlen, and attn_fwd_splitkv with one split): the
    # decode kernel writes the output and the logsumexp itself; 8 x 64 heads
    import torch
    lens_q, lens_k = [1, 1, 1, 0, 1, 1, 1, 1], [2049, 0, 1, 70, 64, 700, 65, 128]
    q, k, v, cu_q, cu_k = _pack(lens_q, lens_k, 64, d, seed=980 + d)
    table = None
    kk, vv = k, v
    if page:
        kk, vv, table = _paginate(k, v, cu_k, lens_k, page, seed=981)
    tq, tk, tv = to_dev(q), to_dev(kk), to_dev(vv)
    tab = None if table is None else _t32(table)
    o1, l1 = lib.fwd_varlen(tq, _t32(cu_q), tk, tv, _t32(cu_k), 1, max(lens_k), causal=True, block_table=tab,
                            page_size=page)
    o2, l2 = lib.fwd_splitkv(tq, _t32(cu_q), tk, tv, _t32(cu_k), 1, max(lens_k), causal=True, block_table=tab,
                             page_size=page, num_splits=1)
    torch.cuda.synchronize()
    o_ref, lse_ref = _reference(q, k, v, cu_q, cu_k, lens_q, lens_k, True)
    assert_close16(to_host(o1), o_ref, l1.cpu().numpy().astype(np.float64), lse_ref, f"one-row whole d{d} page={page}")
    np.testing.assert_array_equal(to_host(o1), to_host(o2))
    np.testing.assert_array_equal(l1.cpu().numpy(), l2.cpu().numpy())
