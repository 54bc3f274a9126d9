"""The C ABI on the CPU (no GPU needed): the shared library loads, exports every
function include/attn.h declares, and rejects every invalid argument with its
status code before anything reaches the device."""
import ctypes
import json
import math
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")
LIB = os.path.join(ROOT, "attention_attn_fwd_10_amd", "libattn_fwd.so")

OK, INVALID, UNSUPPORTED, HIP = 0, 1, 2, 3


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        sys.path.insert(0, ROOT)
        from attention_attn_fwd_10_amd import build
        build.build(verbose=False)
    L = ctypes.CDLL(LIB)
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    I64P = ctypes.POINTER(ctypes.c_int64)
    L.attn_fwd.argtypes = [I, P, I64P, P, I64P, P, I64P, P, I64P, P, I, I, I, I, I, F, I, P]
    L.attn_fp8_quantize.argtypes = [P, I64P, P, P, I, I, I, I, I, P, P]
    L.attn_fwd_fp8.argtypes = [P, P, P, P, P, P, I, P, P, I, I, I, I, I, F, I, P]
    L.attn_fp8_quantize_pow2.argtypes = [P, I64P, P, P, I, I, I, I, I, P, F, P]
    L.attn_fwd_fp8_pow2.argtypes = [P, P, P, P, P, P, I, P, P, I, I, I, I, I, I, P]
    L.attn_bwd.argtypes = [I, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, F, I, P]
    L.attn_int8_quantize.argtypes = [P, I64P, P, P, I, I, I, I, I, P, P]
    L.attn_fwd_int8.argtypes = [P, P, P, P, P, P, I, P, P, I, I, I, I, I, F, I, P]
    L.attn_fwd_varlen.argtypes = [I, P, P, P, P, P, P, I, I, P, P, I, I, I, I, I, I, F, I, P]
    L.attn_fwd_splitkv.argtypes = [I, P, P, P, P, P, P, I, I, P, P, I, I, I, I, I, I, F, I, I, P,
                                   ctypes.c_size_t, P]
    L.attn_fwd_splitkv_noalloc.argtypes = [I, P, P, P, P, P, P, I, I, P, P, I, I, I, I, I, I, F, I, I, P]
    L.attn_fwd_splitkv_workspace_bytes.argtypes = [I, I, I, I]
    I32P = ctypes.POINTER(ctypes.c_int32)
    L.attn_check_indices_host.argtypes = [I32P, I32P, I32P, I, I, I, I, I, I]
    L.attn_set_index_checks.argtypes = [I]
    L.attn_set_index_checks.restype = None
    L.attn_fwd_splitkv_workspace_bytes.restype = ctypes.c_size_t
    L.attn_fwd_bias.argtypes = [I, P, I64P, P, I64P, P, I64P, P, I64P, P, I64P, P, I, I, I, I, I, F, I, P]
    L.attn_status_string.argtypes = [I]
    L.attn_status_string.restype = ctypes.c_char_p
    L.attn_last_error.restype = ctypes.c_char_p
    return L


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("attn_fwd", "attn_fp8_quantize", "attn_fwd_fp8", "attn_fp8_quantize_pow2", "attn_fwd_fp8_pow2",
              "attn_fwd_varlen", "attn_fwd_splitkv",
              "attn_fwd_splitkv_workspace_bytes", "attn_fwd_bias", "attn_int8_quantize", "attn_fwd_int8",
              "attn_bwd", "attn_status_string", "attn_last_error", "attn_fwd_splitkv_noalloc",
              "attn_set_index_checks", "attn_check_indices_host"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if " T " in line)
    for n in declared_functions():
        assert n in exported, n
        assert hasattr(lib, n)


def test_probe_library_exports_its_header():
    """libattn_probe.so (measured ceilings, not on the attention path) exports
    every function include/attn_probe.h declares."""
    path = os.path.join(ROOT, "attention_attn_fwd_10_amd", "libattn_probe.so")
    if not os.path.exists(path):
        sys.path.insert(0, ROOT)
        from attention_attn_fwd_10_amd import build
        build.build(verbose=False)
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "attn_probe.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))
    assert names == ["attn_probe_ceilings", "attn_probe_cycles"]
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if " T " in line)
    for n in names:
        assert n in exported, n


def _s(*v):
    return (ctypes.c_int64 * 3)(*v)


# fake, never dereferenced device addresses (validation fails or returns before use)
A16 = ctypes.c_void_p(0x10000)
A_ODD = ctypes.c_void_p(0x10008)
GOOD = _s(1 << 20, 1024, 128)


def fwd(lib, dtype=0, q=A16, k=A16, v=A16, o=A16, lse=None, B=1, H=1, Sq=1, Sk=1, D=128, scale=0.1, causal=0,
        qs=GOOD, ks=GOOD, vs=GOOD, os_=GOOD):
    return lib.attn_fwd(dtype, q, qs, k, ks, v, vs, o, os_, lse, B, H, Sq, Sk, D, scale, causal, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=2), INVALID),
    (dict(D=96), UNSUPPORTED),
    (dict(D=0), INVALID),
    (dict(B=-1), INVALID),
    (dict(Sk=-3), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(scale=0.0), INVALID),
    (dict(scale=float("inf")), INVALID),
    (dict(causal=2), INVALID),
    (dict(qs=_s(1 << 20, 1024, 12)), INVALID),     # not a multiple of 8 elements
    (dict(ks=_s(-8, 1024, 128)), INVALID),         # negative stride
    (dict(q=None), INVALID),
    (dict(v=None), INVALID),
    (dict(o=A_ODD), INVALID),                      # not 16-byte aligned
    (dict(Sk=4, ks=_s(1 << 20, 64, 128)), INVALID),  # k rows overlap (seq stride < D)
    (dict(vs=_s(1 << 30, 1 << 25, 128)), UNSUPPORTED),  # seq stride above 2^24
    (dict(B=0, q=None, k=None, v=None, o=None), OK),  # empty problem: no-op
    (dict(Sq=0), OK),
])
def test_fwd_validation(lib, kw, status):
    assert fwd(lib, **kw) == status
    if status != OK:
        assert len(lib.attn_last_error()) > 0


def test_null_stride_array(lib):
    assert lib.attn_fwd(0, A16, None, A16, GOOD, A16, GOOD, A16, GOOD, None, 1, 1, 1, 1, 128, 0.1, 0, None) == INVALID


@pytest.mark.parametrize("name", ["attn_fp8_quantize", "attn_int8_quantize"])
def test_quantize_validation(lib, name):
    fn = getattr(lib, name)
    q = lambda **k: fn(k.get("x", A16), k.get("xs", GOOD), k.get("x8", A16), k.get("sc", A16),
                       k.get("B", 1), k.get("H", 1), k.get("S", 1), k.get("D", 128),
                       k.get("br", 128), None, None)
    assert q(br=64) == INVALID
    assert q(D=96) == UNSUPPORTED
    assert q(x=None) == INVALID
    assert q(sc=None) == INVALID
    assert q(S=-1) == INVALID
    assert q(S=0) == OK


def test_quantize_pow2_validation(lib):
    q = lambda **k: lib.attn_fp8_quantize_pow2(A16, GOOD, A16, A16, 1, 1, 1, k.get("D", 128), k.get("br", 128), None,
                                               k.get("pm", 1.0), None)
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert q(pm=bad) == INVALID
    assert q(br=64) == INVALID
    assert q(D=96) == UNSUPPORTED


def test_fp8_pow2_fwd_validation(lib):
    f = lambda **k: lib.attn_fwd_fp8_pow2(A16, A16, A16, A16, A16, A16, k.get("br", 128), A16, None, 1, 1, 1, 1,
                                          k.get("D", 128), k.get("causal", 0), None)
    assert f(D=64) == UNSUPPORTED
    assert f(D=-1) == INVALID
    assert f(br=7) == INVALID
    assert f(causal=5) == INVALID


@pytest.mark.parametrize("name", ["attn_fwd_fp8", "attn_fwd_int8"])
def test_fp8_fwd_validation(lib, name):
    fn = getattr(lib, name)
    f = lambda **k: fn(A16, A16, A16, A16, A16, A16, k.get("br", 128), A16, None, 1, 1, 1, 1,
                       k.get("D", 128), k.get("scale", 0.1), k.get("causal", 0), None)
    assert f(D=64) == UNSUPPORTED
    assert f(D=-1) == INVALID
    assert f(br=7) == INVALID
    assert f(scale=-1.0) == INVALID
    assert f(causal=5) == INVALID


def test_varlen_validation(lib):
    def f(page=64, table=A16, maxp=4, maxk=200, D=128, B=2, total_q=10):
        return lib.attn_fwd_varlen(0, A16, A16, A16, A16, A16, table, maxp, page, A16, None, B, 2, D, total_q, 100,
                                   maxk, 0.1, 1, None)
    assert f(page=48) == INVALID        # not a power of two
    assert f(page=8) == INVALID         # below 16
    assert f(maxp=3, maxk=200) == INVALID  # 3 pages of 64 cannot hold 200 keys
    assert f(maxp=0) == INVALID
    assert f(D=80) == UNSUPPORTED
    assert f(B=0) == OK
    assert f(total_q=0) == OK


def test_splitkv_validation(lib):
    def f(splits=4, ws=A16, ws_bytes=1 << 30, B=2, total_q=10, D=128, page=64, table=A16):
        return lib.attn_fwd_splitkv(0, A16, A16, A16, A16, A16, table, 4, page, A16, None, B, 2, D, total_q, 100,
                                    200, 0.1, 1, splits, ws, ws_bytes, None)
    assert f(splits=0) == INVALID
    assert f(splits=257) == INVALID
    assert f(ws=None) == INVALID                      # workspace needed for splits > 1
    assert f(ws_bytes=1000) == INVALID                # workspace too small
    assert f(ws=A_ODD) == INVALID                     # not 16-byte aligned
    assert f(page=48) == INVALID                      # the varlen checks apply
    assert f(D=80) == UNSUPPORTED
    assert f(B=0) == OK and f(total_q=0) == OK          # empty problems: no-op


def test_splitkv_noalloc_validation(lib):
    def f(splits=4, B=2, total_q=10, H=2, D=128, page=64, table=A16):
        return lib.attn_fwd_splitkv_noalloc(0, A16, A16, A16, A16, A16, table, 4, page, A16, None, B, H, D, total_q,
                                            100, 200, 0.1, 1, splits, None)
    assert f(splits=0) == INVALID
    assert f(splits=257) == INVALID
    assert f(page=48) == INVALID                      # the varlen checks apply
    assert f(D=80) == UNSUPPORTED
    assert f(B=0) == OK and f(total_q=0) == OK          # empty problems: no-op
    # partial results beyond the library's scratch are refused before anything runs
    assert f(splits=16, total_q=4096, H=32) == INVALID
    assert b"scratch" in lib.attn_last_error()


def test_bias_validation(lib):
    def f(D=128, bs=_s(1 << 20, 1024, 64), bias=A16, Sk=4, B=1):
        return lib.attn_fwd_bias(0, A16, GOOD, A16, GOOD, A16, GOOD, bias, bs, A16, GOOD, None, B, 1, 4, Sk, D, 0.1,
                                 0, None)
    assert f(D=256) == UNSUPPORTED
    assert f(bs=_s(1 << 20, 1024, 12)) == INVALID     # row stride not a multiple of 8
    assert f(bs=_s(-8, 0, 8)) == INVALID              # negative stride
    assert f(bias=None) == INVALID
    assert f(bias=A_ODD) == INVALID
    assert f(bs=_s(0, 0, 1 << 29)) == UNSUPPORTED     # a plane beyond 2^31 bytes
    assert f(B=0) == OK


def test_splitkv_workspace_bytes(lib):
    assert lib.attn_fwd_splitkv_workspace_bytes(10, 2, 128, 4) == 4 * 10 * 2 * 129 * 4
    assert lib.attn_fwd_splitkv_workspace_bytes(10, 2, 128, 1) == 0
    assert lib.attn_fwd_splitkv_workspace_bytes(0, 2, 128, 4) == 0


def test_status_strings(lib):
    for code, name in ((0, b"ATTN_OK"), (1, b"ATTN_ERR_INVALID"), (2, b"ATTN_ERR_UNSUPPORTED"),
                       (3, b"ATTN_ERR_HIP"), (99, b"ATTN_STATUS_UNKNOWN")):
        assert lib.attn_status_string(code) == name


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_bwd_validation(lib):
    def f(dtype=0, B=1, H=1, Sq=4, Sk=4, D=128, scale=0.1, causal=0, q=A16, dk=A16, lse=A16):
        return lib.attn_bwd(dtype, q, A16, A16, A16, lse, A16, A16, dk, A16, A16, B, H, Sq, Sk, D, scale, causal,
                            None)
    assert f(D=256) == UNSUPPORTED
    assert f(D=96) == UNSUPPORTED
    assert f(D=0) == INVALID
    assert f(dtype=7) == INVALID
    assert f(scale=0.0) == INVALID
    assert f(causal=2) == INVALID
    assert f(Sq=-1) == INVALID
    assert f(q=None) == INVALID
    assert f(lse=None) == INVALID
    assert f(dk=None) == INVALID
    assert f(B=0) == OK
    assert f(Sq=0, Sk=0) == OK


def test_decode_num_splits():
    import random
    import attention_attn_fwd_10_amd as A
    assert A.decode_num_splits(128, 32768) == 8       # 4 sequences x 32 heads: 1024 waves
    assert A.decode_num_splits(512, 8192) == 2
    assert A.decode_num_splits(32, 131072) == 32
    assert A.decode_num_splits(48, 5000) == 20        # 79 tiles: ranges of 4 tiles, none empty
    assert A.decode_num_splits(4096, 1000) == 1       # enough waves without splitting
    assert A.decode_num_splits(1, 64) == 1
    rng = random.Random(5)
    for _ in range(500):
        nbh, lk = rng.randint(1, 5000), rng.randint(0, 300000)
        s = A.decode_num_splits(nbh, lk)
        tiles = max(1, (lk + 63) // 64)
        per = -(-tiles // s)
        assert 1 <= s <= 256 and (s - 1) * per < tiles   # every range holds keys
        assert s == 1 or per >= 2


def test_auto_num_splits():
    import attention_attn_fwd_10_amd as A
    # decode kernel's rule where the library takes it, the tiled rule elsewhere
    assert A.auto_num_splits(4, 32, 128, 4, 1, 32768, 64) == 8
    assert A.auto_num_splits(4, 32, 128, 4, 1, 32768, 0) == 8
    assert A.auto_num_splits(4, 32, 128, 4, 1, 32768, 16) == 8
    assert A.auto_num_splits(4, 32, 256, 4, 1, 32768, 16) == 8
    assert A.auto_num_splits(4, 32, 128, 4, 1, 32768, 32) == 8
    assert A.auto_num_splits(4, 32, 64, 4, 1, 32768, 0) == 8
    assert A.auto_num_splits(4, 32, 256, 4, 1, 32768, 0) == 8
    assert A.auto_num_splits(4, 32, 128, 8, 2, 32768, 0) == A.splitkv_num_splits(32 * 5, 32768)
    # too few waves for the decode kernel even split: the tiled rule
    assert A.auto_num_splits(1, 8, 128, 1, 1, 1000, 0) == A.splitkv_num_splits(8 * 2, 1000)


def test_splitkv_num_splits_bounds():
    """The split-count rule: between 1 and 16 splits, at least 4 tiles of 64 keys
    in every split the kernel forms (ceil(tiles / splits) each), and no fewer
    splits for fewer work items."""
    import attention_attn_fwd_10_amd as A
    for n_work in (1, 32, 160, 544, 5000):
        for lk in (1, 64, 255, 300, 4096, 32768, 131072, 1 << 20):
            s = A.splitkv_num_splits(n_work, lk)
            tiles = (lk + 63) // 64
            assert 1 <= s <= 16
            per = -(-tiles // s)
            if s > 1:
                assert per >= 4 and tiles - (s - 1) * per >= 1, (n_work, lk, s)
    assert A.splitkv_num_splits(160, 32768) == 16
    assert A.splitkv_num_splits(544, 8192) == 4
    assert A.splitkv_num_splits(32, 131072) >= A.splitkv_num_splits(5000, 131072)


def _i32(vals):
    return (ctypes.c_int32 * len(vals))(*vals) if vals is not None else None


def test_index_check_host(lib):
    """The invariants the varlen kernels rely on, checked on host copies."""
    def f(cq=(0, 3, 3, 10), ck=(0, 5, 9, 9), table=None, maxp=0, page=0, total_q=10, mq=7, mk=5):
        B = len(cq) - 1
        return lib.attn_check_indices_host(_i32(cq), _i32(ck), _i32(table), maxp, page, B, total_q, mq, mk)
    assert f() == OK
    assert f(cq=(1, 3, 3, 10)) == INVALID                 # first query offset not 0
    assert f(ck=(-1, 5, 9, 9)) == INVALID                 # negative key offset
    assert f(cq=(0, 3, 2, 10)) == INVALID                 # decreasing
    assert f(ck=(0, 5, 4, 9)) == INVALID
    assert f(mq=6) == INVALID                             # 7 queries > max_seqlen_q
    assert f(mk=4) == INVALID                             # 5 keys > max_seqlen_k
    assert f(total_q=11) == INVALID                       # cu_seqlens_q[B] != total_q
    assert b"total_q" in lib.attn_last_error()
    # paged: 3 sequences with 5, 4, 0 keys in 4-token pages -> 2, 1, 0 pages
    good = [7, 2, -1, 0, -1, -1, -1, -1, -1]
    assert f(table=good, maxp=3, page=4) == OK            # entries past a sequence's pages are ignored
    assert f(table=[7, -1, -1, 0, -1, -1, -1, -1, -1], maxp=3, page=4) == INVALID   # needed page < 0
    assert b"block_table[0][1]" in lib.attn_last_error()
    assert f(table=[7], maxp=1, page=4) == INVALID        # 2 pages needed, 1 allowed
    assert f(cq=(0,), ck=(0,), total_q=0) == OK           # no sequences
