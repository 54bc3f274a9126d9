"""Python binding of the MI355X fused attention forward library.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libattn_fwd.so``.  torch supplies device memory and the stream.
The entry points mirror the C ABI in ``include/attn.h``:

* ``fwd``            -> ``attn_fwd_ws``         (bf16 / fp16, optional causal mask; the
  workspace for a split tail of the grid, sized by ``attn_fwd_workspace_bytes``)
* ``fp8_quantize``   -> ``attn_fp8_quantize``   (rotation + e4m3 block quantisation)
* ``fwd_fp8``        -> ``attn_fwd_fp8``        (e4m3 forward with per-block scales)
* ``fp8_quantize_pow2`` / ``fwd_fp8_pow2`` -> ``attn_fp8_quantize_pow2`` / ``attn_fwd_fp8_pow2``
  (the same with power-of-two block scales, applied inside the matrix-core
  products; ``fp8_quantize_pow2_q`` codes Q with the softmax scale)
* ``int8_quantize``  -> ``attn_int8_quantize``  (rotation + int8 block quantisation)
* ``fwd_int8``       -> ``attn_fwd_int8``       (int8 scores, e4m3 V and probabilities)
* ``fwd_varlen``     -> ``attn_fwd_varlen``     (packed sequences, optional paged KV)
* ``fwd_splitkv``    -> ``attn_fwd_splitkv``    (keys cut into ranges, merged through the LSEs)
* ``fwd_splitkv_noalloc`` -> ``attn_fwd_splitkv_noalloc`` (the same with the library's own scratch)
* ``bwd``            -> ``attn_bwd``            (dq, dk, dv of the dense forward)

Tensors use the [batch, seq, heads, head_dim] layout (varlen: [tokens, heads,
head_dim]).  If the library has not been built, the first call raises
ImportError: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = ["fwd", "fwd_bias", "fp8_quantize", "fwd_fp8", "fp8_quantize_pow2", "fp8_quantize_pow2_q", "fwd_fp8_pow2",
           "int8_quantize", "fwd_int8", "fwd_varlen", "fwd_splitkv", "fwd_splitkv_noalloc", "bwd",
           "set_index_checks", "lib_path", "AttnError", "ATTN_BF16", "ATTN_FP16", "LOG2E"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libattn_fwd.so")

ATTN_OK, ATTN_ERR_INVALID, ATTN_ERR_UNSUPPORTED, ATTN_ERR_HIP = 0, 1, 2, 3
ATTN_BF16, ATTN_FP16 = 0, 1


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it with `python -m attention_attn_fwd_10_amd.build` "
            "(there is no fallback path)")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    I64P = ctypes.POINTER(ctypes.c_int64)
    lib.attn_fwd.argtypes = [I, P, I64P, P, I64P, P, I64P, P, I64P, P, I, I, I, I, I, F, I, P]
    lib.attn_fwd.restype = I
    lib.attn_fwd_bias.argtypes = [I, P, I64P, P, I64P, P, I64P, P, I64P, P, I64P, P, I, I, I, I, I, F, I, P]
    lib.attn_fwd_bias.restype = I
    lib.attn_fp8_quantize.argtypes = [P, I64P, P, P, I, I, I, I, I, P, P]
    lib.attn_fp8_quantize.restype = I
    lib.attn_fwd_fp8.argtypes = [P, P, P, P, P, P, I, P, P, I, I, I, I, I, F, I, P]
    lib.attn_fwd_fp8.restype = I
    lib.attn_fp8_quantize_pow2.argtypes = [P, I64P, P, P, I, I, I, I, I, P, F, P]
    lib.attn_fp8_quantize_pow2.restype = I
    lib.attn_fwd_fp8_pow2.argtypes = [P, P, P, P, P, P, I, P, P, I, I, I, I, I, I, P]
    lib.attn_fwd_fp8_pow2.restype = I
    lib.attn_bwd.argtypes = [I, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, F, I, P]
    lib.attn_bwd.restype = I
    lib.attn_int8_quantize.argtypes = [P, I64P, P, P, I, I, I, I, I, P, P]
    lib.attn_int8_quantize.restype = I
    lib.attn_fwd_int8.argtypes = [P, P, P, P, P, P, I, P, P, I, I, I, I, I, F, I, P]
    lib.attn_fwd_int8.restype = I
    lib.attn_fwd_varlen.argtypes = [I, P, P, P, P, P, P, I, I, P, P, I, I, I, I, I, I, F, I, P]
    lib.attn_fwd_varlen.restype = I
    SZ = ctypes.c_size_t
    lib.attn_fwd_ws.argtypes = [I, P, I64P, P, I64P, P, I64P, P, I64P, P, I, I, I, I, I, F, I, P, SZ, P]
    lib.attn_fwd_ws.restype = I
    lib.attn_fwd_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    lib.attn_fwd_workspace_bytes.restype = SZ
    lib.attn_fwd_splitkv.argtypes = [I, P, P, P, P, P, P, I, I, P, P, I, I, I, I, I, I, F, I, I, P, SZ, P]
    lib.attn_fwd_splitkv.restype = I
    lib.attn_fwd_splitkv_noalloc.argtypes = [I, P, P, P, P, P, P, I, I, P, P, I, I, I, I, I, I, F, I, I, P]
    lib.attn_fwd_splitkv_noalloc.restype = I
    lib.attn_fwd_splitkv_workspace_bytes.argtypes = [I, I, I, I]
    lib.attn_fwd_splitkv_workspace_bytes.restype = SZ
    lib.attn_set_index_checks.argtypes = [I]
    lib.attn_set_index_checks.restype = None
    lib.attn_status_string.argtypes = [I]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    return lib


class _Library:
    """The loaded ``libattn_fwd.so``, opened at the first call into it, so
    that the build step can import this package before the library exists.
    A call without the library raises ImportError (there is no fallback)."""

    _handle = None

    def __getattr__(self, name):
        if _Library._handle is None:
            _Library._handle = _load()
        return getattr(_Library._handle, name)


_lib = _Library()


def set_index_checks(enable: bool) -> None:
    """Debug switch (process-wide, off by default): the varlen, split-key and
    allocation-free entry points copy cu_seqlens and the block table to the
    host and validate them before launching (attn_set_index_checks)."""
    _lib.attn_set_index_checks(int(bool(enable)))


def _check(status: int):
    if status != ATTN_OK:
        msg = _lib.attn_last_error().decode() or _lib.attn_status_string(status).decode()
        raise AttnError(status, msg)


def _strides(t):
    """[B, S, H, D] element strides as the C ABI's {batch, seq, head} triple."""
    if t.stride(3) != 1:
        raise ValueError("head_dim must be the contiguous dimension")
    arr = (ctypes.c_int64 * 3)(t.stride(0), t.stride(1), t.stride(2))
    return arr


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dtype_code(dt):
    import torch
    if dt == torch.bfloat16:
        return ATTN_BF16
    if dt == torch.float16:
        return ATTN_FP16
    raise TypeError(f"unsupported dtype {dt}: bf16 or fp16 expected")


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must live on the GPU")


def _require(t, name, shape, dtype, contiguous=True):
    """The C ABI sees only pointers: a tensor of another shape, dtype or
    layout would be misread on the device, so it is refused here."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _scale_shape(B, H, S, block_rows):
    return (B, H, (S + 127) // 128) if block_rows else (1,)


def fwd(q, k, v, softmax_scale=None, causal=False, out=None, lse=None, return_lse=True, stream=None,
        workspace=None):
    """Fused attention forward.  q [B, Sq, H, D], k/v [B, Sk, H, D] (bf16 or
    fp16, head_dim contiguous).  The fp32 workspace of a split grid tail is
    allocated here (through torch's allocator) unless given.  Returns
    (o [B, Sq, H, D], lse [B, H, Sq] fp32)."""
    import torch
    _require_cuda(q, k, v, out, lse, workspace)
    B, Sq, H, D = q.shape
    Sk = k.shape[1]
    if k.shape != (B, Sk, H, D) or v.shape != (B, Sk, H, D):
        raise ValueError("k and v must be [B, Sk, H, D] matching q")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share a dtype")
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format) if not q.is_contiguous() \
            else torch.empty_like(q)
    else:
        _require(out, "out", (B, Sq, H, D), q.dtype, contiguous=False)
    if lse is None and return_lse:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _require(lse, "lse", (B, H, Sq), torch.float32)
    with torch.cuda.device(q.device):
        need = int(_lib.attn_fwd_workspace_bytes(_dtype_code(q.dtype), B, H, Sq, Sk, D, int(bool(causal))))
        if workspace is None and need > 0:
            workspace = torch.empty(need // 4, dtype=torch.float32, device=q.device)
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        _check(_lib.attn_fwd_ws(_dtype_code(q.dtype), _ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v),
                                _strides(v), _ptr(out), _strides(out), _ptr(lse), B, H, Sq, Sk, D, scale,
                                int(bool(causal)), _ptr(workspace), ws_bytes, _stream(stream)))
    return out, lse


def pad_bias(bias):
    """Copy a [B, H, Sq, Sk] bias into storage whose key rows are padded to a
    multiple of 8 elements (the layout fwd_bias needs); returns the padded
    view."""
    import torch
    B, H, Sq, Sk = bias.shape
    pitch = -(-Sk // 8) * 8
    buf = torch.zeros((B, H, Sq, pitch), dtype=bias.dtype, device=bias.device)
    buf[..., :Sk] = bias
    return buf[..., :Sk]


def fwd_bias(q, k, v, bias, softmax_scale=None, causal=False, out=None, lse=None, stream=None):
    """Fused attention forward with an additive score bias: s = scale <q, k> +
    bias[b, h, i, j].  bias is [B, H, Sq, Sk] of q's dtype (any of its first
    three dims may be broadcast with stride 0); its key dim must be contiguous
    and its other strides multiples of 8 (see pad_bias).  Returns (o, lse)."""
    import torch
    _require_cuda(q, k, v, bias, out, lse)
    B, Sq, H, D = q.shape
    Sk = k.shape[1]
    if k.shape != (B, Sk, H, D) or v.shape != (B, Sk, H, D):
        raise ValueError("k and v must be [B, Sk, H, D] matching q")
    if not (q.dtype == k.dtype == v.dtype == bias.dtype):
        raise TypeError("q, k, v and bias must share a dtype")
    if bias.dim() != 4 or bias.shape[3] != Sk or any(bias.shape[i] not in (1, n) for i, n in enumerate((B, H, Sq))):
        raise ValueError("bias must broadcast to [B, H, Sq, Sk]")
    if Sk > 1 and bias.stride(3) != 1:
        raise ValueError("bias keys must be contiguous")
    bst = [0 if bias.shape[i] == 1 else bias.stride(i) for i in range(3)]
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format) if not q.is_contiguous() \
            else torch.empty_like(q)
    else:
        _require(out, "out", (B, Sq, H, D), q.dtype, contiguous=False)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    else:
        _require(lse, "lse", (B, H, Sq), torch.float32)
    _check(_lib.attn_fwd_bias(_dtype_code(q.dtype), _ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v),
                              _strides(v), _ptr(bias), (ctypes.c_int64 * 3)(*bst), _ptr(out), _strides(out),
                              _ptr(lse), B, H, Sq, Sk, D, scale, int(bool(causal)), _stream(stream)))
    return out, lse


def _quantize(fn, code_dtype, x, block_rows, signs, out, scales, stream, premul=None):
    import torch
    _require_cuda(x, signs, out, scales)
    if x.dtype != torch.bfloat16:
        raise TypeError("the 8-bit quantisers expect bf16 input")
    B, S, H, D = x.shape
    if out is None:
        out = torch.empty((B, S, H, D), dtype=code_dtype, device=x.device)
    elif out.dtype != code_dtype or not out.is_contiguous() or out.shape != x.shape:
        raise ValueError(f"out must be a contiguous {code_dtype} tensor shaped like x")
    if scales is None:
        scales = torch.empty(_scale_shape(B, H, S, block_rows), dtype=torch.float32, device=x.device)
    else:
        _require(scales, "scales", _scale_shape(B, H, S, block_rows), torch.float32)
    if signs is not None and (signs.dtype != torch.int8 or signs.numel() != D):
        raise ValueError("signs must be int8 [D]")
    extra = () if premul is None else (float(premul),)
    _check(fn(_ptr(x), _strides(x), _ptr(out), _ptr(scales), B, H, S, D, int(block_rows), _ptr(signs), *extra,
              _stream(stream)))
    return out, scales


def fp8_quantize(x, block_rows=128, signs=None, out=None, scales=None, stream=None):
    """Quantise a bf16 [B, S, H, D] tensor to e4m3 (uint8 codes) with one scale
    per (b, h, 128-row block) or per tensor (block_rows=0), optionally after the
    random-sign Hadamard rotation given by ``signs`` (int8 [D] of +-1)."""
    import torch
    return _quantize(_lib.attn_fp8_quantize, torch.uint8, x, block_rows, signs, out, scales, stream)


LOG2E = 1.4426950408889634


def fp8_quantize_pow2(x, block_rows=128, signs=None, premul=1.0, out=None, scales=None, stream=None):
    """``fp8_quantize`` with power-of-two scales (the smallest power of two at
    or above amax / 448), every value multiplied by ``premul`` first: the input
    form of ``fwd_fp8_pow2`` (premul 1 for K and V; Q: ``fp8_quantize_pow2_q``)."""
    import torch
    return _quantize(_lib.attn_fp8_quantize_pow2, torch.uint8, x, block_rows, signs, out, scales, stream, premul)


def fp8_quantize_pow2_q(q, softmax_scale=None, block_rows=128, signs=None, out=None, scales=None, stream=None):
    """``fp8_quantize_pow2`` of a query tensor: premul = softmax_scale * log2(e)
    (softmax_scale defaults to 1/sqrt(head_dim))."""
    scale = 1.0 / math.sqrt(q.shape[-1]) if softmax_scale is None else float(softmax_scale)
    return fp8_quantize_pow2(q, block_rows, signs, scale * LOG2E, out, scales, stream)


def int8_quantize(x, block_rows=128, signs=None, out=None, scales=None, stream=None):
    """Quantise a bf16 [B, S, H, D] tensor to symmetric int8 codes (scale =
    amax / 127) per (b, h, 128-row block) or per tensor, optionally after the
    random-sign Hadamard rotation."""
    import torch
    return _quantize(_lib.attn_int8_quantize, torch.int8, x, block_rows, signs, out, scales, stream)


def _check_8bit(q8, q_scale, k8, k_scale, v8, v_scale, block_rows, out, lse, qk_dtype):
    """Shapes, dtypes and layouts of the 8-bit forward's operands: q8 and k8
    codes of qk_dtype, v8 e4m3 codes (uint8), all contiguous [B, S, H, D];
    float32 scales [B, H, ceil(S/128)] (block_rows 128) or [1] (0)."""
    import torch
    if block_rows not in (0, 128):
        raise ValueError("block_rows must be 128 or 0")
    B, Sq, H, D = q8.shape
    Sk = k8.shape[1]
    _require(q8, "q8", (B, Sq, H, D), qk_dtype)
    _require(k8, "k8", (B, Sk, H, D), qk_dtype)
    _require(v8, "v8", (B, Sk, H, D), torch.uint8)
    _require(q_scale, "q_scale", _scale_shape(B, H, Sq, block_rows), torch.float32)
    _require(k_scale, "k_scale", _scale_shape(B, H, Sk, block_rows), torch.float32)
    _require(v_scale, "v_scale", _scale_shape(B, H, Sk, block_rows), torch.float32)
    if out is not None:
        _require(out, "out", (B, Sq, H, D), torch.bfloat16)
    if lse is not None:
        _require(lse, "lse", (B, H, Sq), torch.float32)


def fwd_fp8(q8, q_scale, k8, k_scale, v8, v_scale, block_rows=128, softmax_scale=None, causal=False,
            out=None, lse=None, stream=None):
    """8-bit fused forward on e4m3 codes (uint8 [B, S, H, D], contiguous) and
    their scales.  Returns (o bf16 [B, Sq, H, D], lse fp32 [B, H, Sq])."""
    import torch
    _require_cuda(q8, q_scale, k8, k_scale, v8, v_scale, out, lse)
    B, Sq, H, D = q8.shape
    Sk = k8.shape[1]
    _check_8bit(q8, q_scale, k8, k_scale, v8, v_scale, block_rows, out, lse, torch.uint8)
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty((B, Sq, H, D), dtype=torch.bfloat16, device=q8.device)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q8.device)
    _check(_lib.attn_fwd_fp8(_ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale), _ptr(v8), _ptr(v_scale),
                             int(block_rows), _ptr(out), _ptr(lse), B, H, Sq, Sk, D, scale, int(bool(causal)),
                             _stream(stream)))
    return out, lse


def fwd_fp8_pow2(q8, q_scale, k8, k_scale, v8, v_scale, block_rows=128, causal=False, out=None, lse=None,
                 stream=None):
    """``fwd_fp8`` on the power-of-two form (``fp8_quantize_pow2``; the Q codes
    carry the softmax scale, so there is no softmax_scale argument).  Returns
    (o bf16 [B, Sq, H, D], lse fp32 [B, H, Sq])."""
    import torch
    _require_cuda(q8, q_scale, k8, k_scale, v8, v_scale, out, lse)
    B, Sq, H, D = q8.shape
    Sk = k8.shape[1]
    _check_8bit(q8, q_scale, k8, k_scale, v8, v_scale, block_rows, out, lse, torch.uint8)
    if out is None:
        out = torch.empty((B, Sq, H, D), dtype=torch.bfloat16, device=q8.device)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q8.device)
    _check(_lib.attn_fwd_fp8_pow2(_ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale), _ptr(v8), _ptr(v_scale),
                                  int(block_rows), _ptr(out), _ptr(lse), B, H, Sq, Sk, D, int(bool(causal)),
                                  _stream(stream)))
    return out, lse


def fwd_int8(q8, q_scale, k8, k_scale, v8, v_scale, block_rows=128, softmax_scale=None, causal=False,
             out=None, lse=None, stream=None):
    """Fused forward with int8 scores: q8, k8 int8 codes and v8 e4m3 codes
    (uint8), all [B, S, H, D] contiguous, with their scales.  Returns
    (o bf16 [B, Sq, H, D], lse fp32 [B, H, Sq])."""
    import torch
    _require_cuda(q8, q_scale, k8, k_scale, v8, v_scale, out, lse)
    B, Sq, H, D = q8.shape
    Sk = k8.shape[1]
    _check_8bit(q8, q_scale, k8, k_scale, v8, v_scale, block_rows, out, lse, torch.int8)
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty((B, Sq, H, D), dtype=torch.bfloat16, device=q8.device)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q8.device)
    _check(_lib.attn_fwd_int8(_ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale), _ptr(v8), _ptr(v_scale),
                              int(block_rows), _ptr(out), _ptr(lse), B, H, Sq, Sk, D, scale, int(bool(causal)),
                              _stream(stream)))
    return out, lse


def _check_varlen(q, cu_seqlens_q, k, v, cu_seqlens_k, block_table, page_size, out, lse):
    """Operands of the packed / paged forward: q [total_q, H, D]; k, v of q's
    dtype, packed [total_k, H, D] or paged [num_pages, page_size, H, D]; int32
    cu_seqlens [B+1] and block table [B, max_pages]; out and lse shaped like
    the results.  Returns B and max_pages."""
    import torch
    total_q, H, D = q.shape
    B = cu_seqlens_q.numel() - 1
    for t in (q, k, v):
        if not t.is_contiguous():
            raise ValueError("varlen tensors must be contiguous")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share a dtype")
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    for t in (cu_seqlens_q, cu_seqlens_k):
        if t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous():
            raise TypeError("cu_seqlens must be contiguous 1-d int32")
    if cu_seqlens_k.numel() != B + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both have B + 1 entries")
    max_pages = 0
    if block_table is not None:
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or not block_table.is_contiguous():
            raise ValueError("block_table must be contiguous int32 [B, max_pages]")
        if block_table.shape[0] != B:
            raise ValueError("block_table must have one row per sequence")
        max_pages = block_table.shape[1]
        if k.dim() != 4 or k.shape[1] != page_size or tuple(k.shape[2:]) != (H, D):
            raise ValueError("paged k/v must be [num_pages, page_size, H, D]")
    elif k.dim() != 3 or tuple(k.shape[1:]) != (H, D):
        raise ValueError("packed k/v must be [total_k, H, D]")
    if out is not None:
        _require(out, "out", (total_q, H, D), q.dtype)
    if lse is not None:
        _require(lse, "lse", (H, total_q), torch.float32)
    return B, max_pages


def fwd_varlen(q, cu_seqlens_q, k, v, cu_seqlens_k, max_seqlen_q, max_seqlen_k, softmax_scale=None,
               causal=False, block_table=None, page_size=0, out=None, lse=None, stream=None):
    """Packed variable-length forward.  q [total_q, H, D]; cu_seqlens int32
    [B+1] on the device.  Without a block table k, v are packed [total_k, H, D];
    with one they are paged caches [num_pages, page_size, H, D].  Returns
    (o [total_q, H, D], lse fp32 [H, total_q])."""
    import torch
    _require_cuda(q, cu_seqlens_q, k, v, cu_seqlens_k, block_table, out, lse)
    total_q, H, D = q.shape
    B, max_pages = _check_varlen(q, cu_seqlens_q, k, v, cu_seqlens_k, block_table, page_size, out, lse)
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((H, total_q), dtype=torch.float32, device=q.device)
    _check(_lib.attn_fwd_varlen(_dtype_code(q.dtype), _ptr(q), _ptr(cu_seqlens_q), _ptr(k), _ptr(v),
                                _ptr(cu_seqlens_k), _ptr(block_table), max_pages, int(page_size), _ptr(out),
                                _ptr(lse), B, H, D, total_q, int(max_seqlen_q), int(max_seqlen_k), scale,
                                int(bool(causal)), _stream(stream)))
    return out, lse


def splitkv_num_splits(n_work, max_seqlen_k, target=2048, min_tiles=4, max_splits=16):
    """A split count for attn_fwd_splitkv: about `target` workgroups (n_work
    tiles x splits), with the 64-key tiles per split rounded down to a power of
    two (at least `min_tiles`) and at most `max_splits` splits.  Measured on
    one-query decoding over 64-token paged caches (32 heads, d128): 4 x 32768
    keys 16 splits 5.28 TB/s (7 splits: 4.57), 16 x 8192 keys 4 splits 5.33
    (2 splits: 4.70), 1 x 131072 keys 16 splits 3.65."""
    tiles = max(1, (int(max_seqlen_k) + 63) // 64)
    want = max(1, -(-int(target) // max(1, int(n_work))))
    per = max(1, -(-tiles // want))
    per = max(int(min_tiles), 1 << (per.bit_length() - 1))
    return int(max(1, min(-(-tiles // per), tiles // int(min_tiles), max_splits)))


def decode_num_splits(n_seq_heads, max_seqlen_k, target=1024, min_tiles=2, max_splits=256):
    """A split count for one query row per sequence (the
    streaming decode kernel, one wave per sequence, key range and head): about
    `target` waves (n_seq_heads x splits; one per SIMD of the chip), at least
    `min_tiles` 64-key tiles per range and no empty range.  Measured on
    one-query decoding (d128): 4 x 32 heads x 32768 keys 8 splits 5.91 TB/s (16:
    5.75), 16 x 32 x 8192 2 splits 5.92 (4: 5.82), 1 x 32 x 131072 32 splits
    5.59 (64: 5.22), 64 x 8 x 4096 2 splits 5.25 (4: 4.83)."""
    tiles = max(1, (int(max_seqlen_k) + 63) // 64)
    want = max(1, -(-int(target) // max(1, int(n_seq_heads))))
    splits = max(1, min(want, tiles // int(min_tiles), int(max_splits)))
    per = -(-tiles // splits)
    return int(-(-tiles // per))


DECODE_MIN_WAVES = 512  # fewest (sequence, key range, head) items the library runs on the decode kernel


def auto_num_splits(B, H, D, total_q, max_seqlen_q, max_seqlen_k, page_size=0):
    """The split count fwd_splitkv takes when none is given: the decode rule
    when the library runs the decode kernel (one query row per sequence, a
    packed or paged cache, enough waves), else the
    tiled kernel's rule."""
    if int(max_seqlen_q) == 1 and int(D) in (64, 128, 256):
        splits = decode_num_splits(int(B) * int(H), max_seqlen_k)
        if int(B) * int(H) * splits >= DECODE_MIN_WAVES:
            return splits
    n_work = int(H) * (-(-int(total_q) // 128) + int(B))
    return splitkv_num_splits(n_work, max_seqlen_k)


def fwd_splitkv(q, cu_seqlens_q, k, v, cu_seqlens_k, max_seqlen_q, max_seqlen_k, softmax_scale=None,
                causal=False, block_table=None, page_size=0, num_splits=None, out=None, lse=None,
                workspace=None, stream=None):
    """fwd_varlen with each sequence's keys cut into num_splits ranges that run
    as separate work items, then merged through their logsumexps (for short
    queries over long key caches).  num_splits=None picks a count from the
    problem size.  The fp32 workspace is allocated here unless given.
    Returns (o [total_q, H, D], lse fp32 [H, total_q])."""
    import torch
    _require_cuda(q, cu_seqlens_q, k, v, cu_seqlens_k, block_table, out, lse, workspace)
    total_q, H, D = q.shape
    B, max_pages = _check_varlen(q, cu_seqlens_q, k, v, cu_seqlens_k, block_table, page_size, out, lse)
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if num_splits is None:
        num_splits = auto_num_splits(B, H, D, total_q, max_seqlen_q, max_seqlen_k,
                                     page_size if block_table is not None else 0)
    num_splits = int(num_splits)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((H, total_q), dtype=torch.float32, device=q.device)
    need = int(_lib.attn_fwd_splitkv_workspace_bytes(total_q, H, D, num_splits))
    if workspace is None and need > 0:
        workspace = torch.empty(need // 4, dtype=torch.float32, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.attn_fwd_splitkv(_dtype_code(q.dtype), _ptr(q), _ptr(cu_seqlens_q), _ptr(k), _ptr(v),
                                 _ptr(cu_seqlens_k), _ptr(block_table), max_pages, int(page_size), _ptr(out),
                                 _ptr(lse), B, H, D, total_q, int(max_seqlen_q), int(max_seqlen_k), scale,
                                 int(bool(causal)), num_splits, _ptr(workspace), ws_bytes, _stream(stream)))
    return out, lse


def fwd_splitkv_noalloc(q, cu_seqlens_q, k, v, cu_seqlens_k, max_seqlen_q, max_seqlen_k, out, lse,
                        num_splits, softmax_scale=None, causal=False, block_table=None, page_size=0, stream=None):
    """fwd_splitkv for callers that cannot allocate: the partial results go to
    the library's per-device scratch (attn_fwd_splitkv_noalloc), and the caller
    passes the outputs, out [total_q, H, D] and lse fp32 [H, total_q] (or
    None).  Calls that overlap on one device race on that scratch."""
    _require_cuda(q, cu_seqlens_q, k, v, cu_seqlens_k, block_table, out, lse)
    total_q, H, D = q.shape
    B, max_pages = _check_varlen(q, cu_seqlens_q, k, v, cu_seqlens_k, block_table, page_size, out, lse)
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    _check(_lib.attn_fwd_splitkv_noalloc(_dtype_code(q.dtype), _ptr(q), _ptr(cu_seqlens_q), _ptr(k), _ptr(v),
                                         _ptr(cu_seqlens_k), _ptr(block_table), max_pages, int(page_size),
                                         _ptr(out), _ptr(lse), B, H, D, total_q, int(max_seqlen_q),
                                         int(max_seqlen_k), scale, int(bool(causal)), int(num_splits),
                                         _stream(stream)))
    return out, lse


def bwd(q, k, v, o, lse, dout, softmax_scale=None, causal=False, dq=None, dk=None, dv=None, workspace=None,
        stream=None):
    """Gradients of ``fwd``: q, o, dout [B, Sq, H, D], k, v [B, Sk, H, D] (bf16
    or fp16, contiguous), lse fp32 [B, H, Sq] from the forward.  Returns
    (dq, dk, dv)."""
    import torch
    _require_cuda(q, k, v, o, lse, dout, dq, dk, dv, workspace)
    B, Sq, H, D = q.shape
    Sk = k.shape[1]
    for t in (q, k, v, o, dout):
        if not t.is_contiguous() or t.dtype != q.dtype:
            raise ValueError("q, k, v, o and dout must be contiguous and share a dtype")
    if k.shape != (B, Sk, H, D) or v.shape != k.shape or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("shapes must be q/o/dout [B, Sq, H, D] and k/v [B, Sk, H, D]")
    if lse.dtype != torch.float32 or lse.shape != (B, H, Sq) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, H, Sq]")
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _require(dq, "dq", q.shape, q.dtype)
    _require(dk, "dk", k.shape, q.dtype)
    _require(dv, "dv", v.shape, q.dtype)
    if workspace is None:
        workspace = torch.empty((2, B, H, Sq), dtype=torch.float32, device=q.device)
    elif workspace.dtype != torch.float32 or workspace.numel() < 2 * B * H * Sq or not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous float32 with at least 2 * B * H * Sq elements")
    _check(_lib.attn_bwd(_dtype_code(q.dtype), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                         _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), B, H, Sq, Sk, D, scale, int(bool(causal)),
                         _stream(stream)))
    return dq, dk, dv
