"""GPU parity of the wide dense forward (256-row workgroups) and of its split
tail: when the grid's last round is partial, attn_fwd_ws runs that round's
work items as key ranges and merges them through their logsumexps (head dim
128, 4096 keys or more; head dim 64 runs 128-row workgroups and takes no
workspace).

Shapes are derived from the device's compute-unit count so that the grid has
the intended tail: one (batch, head) plane more than whole rounds, with a
ragged last query block and key counts that leave a partial last key tile.
Every row of the split work items is compared with the float64 oracle, plus
sampled rows of the others."""
import math

import numpy as np
import pytest

import workloads as W
from oracle import attention as OA
from tests.parity import assert_close16, sample_rows, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_attn_fwd_10_amd as A
    return A


def _cus():
    import torch
    return torch.cuda.get_device_properties(0).multi_processor_count


def _rows_ref(q, k, v, scale, b, h, rows):
    return OA.naive_head(q[b, rows, h], k[b, :, h], v[b, :, h], scale, False, rows=rows, lq=q.shape[1])


def _check_rows(o, lse, q, k, v, scale, b, h, rows, what, dtype="bf16"):
    import torch
    idx = torch.as_tensor(rows, device=o.device)
    oo = o[b, idx, h].float().cpu().numpy().astype(np.float64)[None, :, None]
    ll = lse[b, h, idx].cpu().numpy().astype(np.float64)[None, None]
    o_ref, l_ref = _rows_ref(q, k, v, scale, b, h, rows)
    return assert_close16(oo, o_ref[None, :, None], ll, l_ref[None, None], what, dtype=dtype)


@pytest.mark.parametrize("d", [128])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("sk", [None, 4100])
def test_split_tail(lib, d, dtype, sk):
    import torch
    cus = _cus()
    if cus % 8:
        pytest.skip(f"{cus} compute units: the shape below assumes a multiple of 8")
    H, rows_per = 8, 256
    nq = cus // H + 1                # H * nq = cus + 8 work items: a tail of 8
    sq = rows_per * nq - 100         # ragged last query block
    sk = sq if sk is None else sk    # 4100 keys: 65 tiles, the last one of 4 keys
    need = lib._lib.attn_fwd_workspace_bytes(0 if dtype == "bf16" else 1, 1, H, sq, sk, d, 0)
    splits = min(8, cus // 8)
    tiles = -(-sk // 64)
    per = -(-tiles // splits)
    splits = -(-tiles // per)
    assert need == splits * 8 * rows_per * (d + 1) * 4
    q, k, v = W.qkv_normal(7000 + d + sk, (1, sq, H, d), (1, sk, H, d))
    if dtype == "fp16":  # values the fp16 inputs hold exactly
        q, k, v = (W.f16_round(x).astype(np.float32) for x in (q, k, v))
    scale = 1 / math.sqrt(d)
    o, lse = lib.fwd(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), causal=False)
    torch.cuda.synchronize()
    # the split work items are the last 8 logical tiles: head 7, query blocks nq-8 .. nq-1
    tail_rows = np.arange(rows_per * (nq - 8), sq)
    print(_check_rows(o, lse, q, k, v, scale, 0, H - 1, tail_rows, f"tail d{d} {dtype} sk{sk}", dtype))
    rows = sample_rows(sq, seed=d + sk, n_random=16)
    for h in (0, 3, H - 1):
        _check_rows(o, lse, q, k, v, scale, 0, h, rows, f"whole d{d} {dtype} sk{sk} h{h}", dtype)
    # the same call again gives the same bits (no ordering between the splits)
    o2, lse2 = lib.fwd(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), causal=False)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_split_tail_workspace_checks(lib):
    import torch
    cus = _cus()
    H, d = 8, 128
    sq = 256 * (cus // H + 1)
    q, k, v = (to_dev(x) for x in W.qkv_normal(71, (1, sq, H, d)))
    need = lib._lib.attn_fwd_workspace_bytes(0, 1, H, sq, sq, d, 0)
    if need == 0:
        pytest.skip("no split tail on this device")
    small = torch.empty(need // 4 - 1, dtype=torch.float32, device="cuda")
    with pytest.raises(lib.AttnError):
        lib.fwd(q, k, v, workspace=small)
    # a caller-given workspace of the right size gives the same result as the
    # one the binding allocates
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda")
    o1, l1 = lib.fwd(q, k, v, workspace=ws)
    o2, l2 = lib.fwd(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_d64_takes_no_workspace(lib):
    """Head dim 64 runs its 128-row workgroups at any length: no split tail,
    so no workspace, and a given one changes nothing."""
    import torch
    cus = _cus()
    H, d = 8, 64
    sq = 256 * (cus // H + 1)
    assert lib._lib.attn_fwd_workspace_bytes(0, 1, H, sq, sq, d, 0) == 0
    q, k, v = W.qkv_normal(72, (1, sq, H, d))
    ws = torch.zeros(1024, dtype=torch.float32, device="cuda")
    o1, l1 = lib.fwd(to_dev(q), to_dev(k), to_dev(v), workspace=ws)
    o2, l2 = lib.fwd(to_dev(q), to_dev(k), to_dev(v))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    rows = sample_rows(sq, seed=5, n_random=16)
    _check_rows(o1, l1, q, k, v, 1 / math.sqrt(d), 0, 3, rows, "d64 no workspace")


@pytest.mark.parametrize("d", [128])
def test_whole_rounds(lib, d):
    """A grid of exactly one round of 256-row work items: the wide layout
    without a split (no workspace)."""
    import torch
    cus = _cus()
    H = 8
    sq = 256 * (cus // H)
    if lib._lib.attn_fwd_workspace_bytes(0, 1, H, sq, sq, d, 0) != 0:
        pytest.skip("unexpected split on this device")
    q, k, v = W.qkv_normal(8000 + d, (1, sq, H, d))
    o, lse = lib.fwd(to_dev(q), to_dev(k), to_dev(v), causal=False)
    torch.cuda.synchronize()
    rows = sample_rows(sq, seed=d, n_random=24)
    for h in range(H):
        _check_rows(o, lse, q, k, v, 1 / math.sqrt(d), 0, h, rows, f"whole rounds d{d} h{h}")
