"""GPU test of the allocation-free split-key entry point
(attn_fwd_splitkv_noalloc, called through the C ABI by the binding): its
output equals attn_fwd_splitkv's with a caller-allocated workspace, bit for
bit, on two calls in a row whose second input is smaller (the scratch keeps
the first call's contents), and both match the float64 oracle."""
import math

import numpy as np
import pytest

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


def _case(lib, lens_q, lens_k, H, d, splits, causal, seed, page=0):
    import torch
    q, k, v, cu_q, cu_k = _pack(lens_q, lens_k, H, d, seed)
    table = None
    if page:
        k, v, table = _paginate(k, v, cu_k, lens_k, page, seed + 1)
    tq, tk, tv = to_dev(q), to_dev(k), to_dev(v)
    tcq, tck = _t32(cu_q), _t32(cu_k)
    ttab = None if table is None else _t32(table)
    mq, mk = int(max(lens_q)), int(max(lens_k))
    o_ws, lse_ws = lib.fwd_splitkv(tq, tcq, tk, tv, tck, mq, mk, causal=causal, block_table=ttab,
                                   page_size=page, num_splits=splits)
    o_na = torch.full_like(o_ws, float("nan"))
    lse_na = torch.full_like(lse_ws, float("nan"))
    lib.fwd_splitkv_noalloc(tq, tcq, tk, tv, tck, mq, mk, o_na, lse_na, splits, causal=causal,
                            block_table=ttab, page_size=page)
    torch.cuda.synchronize()
    assert torch.equal(o_na, o_ws) and torch.equal(lse_na, lse_ws)
    if page:
        # the oracle works on the packed layout
        q, k, v, cu_q, cu_k = _pack(lens_q, lens_k, H, d, seed)
    o_ref, lse_ref = OA.attention_varlen(q, cu_q, k, v, cu_k, 1 / math.sqrt(d), causal)
    assert_close16(to_host(o_na), o_ref, lse_na.cpu().numpy().astype(np.float64), lse_ref,
                   f"noalloc d{d} splits={splits} causal={causal}")


def test_two_calls_second_smaller(lib):
    # first call: 4 sequences, up to 3 queries each over up to 5000 keys, 8
    # heads, d128, 16 splits, 64-token pages; second: fewer, shorter, d64
    _case(lib, [1, 3, 2, 1], [5000, 700, 64, 3100], 8, 128, 16, False, 300, page=64)
    _case(lib, [1, 2], [900, 130], 2, 64, 4, True, 310)


def test_oversized_request_is_refused(lib):
    import torch
    A = lib
    total_q, H, D, splits = 4096, 32, 128, 16
    assert A._lib.attn_fwd_splitkv_workspace_bytes(total_q, H, D, splits) > 32 << 20
    q = torch.zeros((total_q, H, D), dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, total_q], dtype=torch.int32, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((H, total_q), dtype=torch.float32, device="cuda")
    with pytest.raises(A.AttnError, match="scratch"):
        A.fwd_splitkv_noalloc(q, cu, q, q, cu, total_q, total_q, o, lse, splits)
