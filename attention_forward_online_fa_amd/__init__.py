"""Fused attention forward pass for AMD MI355X (gfx950).

Thin Python binding over the C ABI in ``include/fa.h`` (``libfa.so``). Every
step of the computation runs in the library's HIP kernels; this module only
checks and marshals arguments. torch provides device memory and streams.

    o, lse = fwd(q, k, v, causal=True, window=0)

q: [B, H, Sq, D], k and v: [B, HKV, Sk, D] CUDA (HIP) tensors of dtype
float32, bfloat16 or float16; o has q's shape and dtype, lse is float32
[B, H, Sq] in natural-log units. A row with no visible key gets o = 0 and
lse = -inf. Contiguous tensors go through fa_fwd_ex; any other strides with a
contiguous last dimension (e.g. token-major [B, S, H, D] storage viewed as
[B, H, S, D] with ``.transpose(1, 2)``, or slices of packed QKV) through
fa_fwd_strided, which checks the stride rules of include/fa.h. A block mask
(``block_mask=``, uint8 or bool [1 or B, 1 or HKV or H, ceil(Sq/128),
ceil(Sk/64)] on the device) runs fa_fwd_block_sparse.
"""
from __future__ import annotations

import ctypes
import math

from ._lib import (FA_BF16, FA_F16, FA_F32, FA_MASK_BLOCK_K, FA_MASK_BLOCK_Q, FA_MAX_SPLITS,
                   FaError, lib, library_path)

__all__ = ["fwd", "fwd_into", "fwd_noalloc_into", "bwd", "plan_splits", "bwd_plan",
           "schedule_table", "release", "FaError",
           "library_path", "default_scale", "FA_F32", "FA_BF16", "FA_F16", "FA_MAX_SPLITS",
           "FA_MASK_BLOCK_Q", "FA_MASK_BLOCK_K"]


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return FA_F32
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float16:
        return FA_F16
    raise TypeError(f"unsupported dtype {t.dtype}: use float32, bfloat16 or float16")


_DTYPE_NAMES = {"f32": FA_F32, "bf16": FA_BF16, "f16": FA_F16}


def _dtype_name_code(dtype) -> int:
    if dtype in _DTYPE_NAMES.values():
        return int(dtype)
    if dtype in _DTYPE_NAMES:
        return _DTYPE_NAMES[dtype]
    raise TypeError(f"unknown dtype {dtype!r}: use 'f32', 'bf16' or 'f16'")


def default_scale(D: int) -> float:
    """1/sqrt(D) rounded to float32, the value the library receives."""
    import numpy as np
    return float(np.float32(1.0 / math.sqrt(D)))


def _check(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [B, heads, S, D]")
        if t.stride(3) != 1 and t.shape[3] > 1:
            raise ValueError(f"{name}: the head dimension must be contiguous (stride 1)")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share one dtype")
    if k.shape != v.shape or q.shape[0] != k.shape[0] or q.shape[3] != k.shape[3]:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")


def _check_mask(block_mask, B, H, HKV, Sq, Sk, q):
    import torch
    if not block_mask.is_cuda or block_mask.device != q.device:
        raise ValueError("block_mask must be on q's device")
    if block_mask.dtype not in (torch.uint8, torch.bool) or not block_mask.is_contiguous():
        raise ValueError("block_mask must be a contiguous uint8 or bool tensor")
    nqb = -(-Sq // FA_MASK_BLOCK_Q)
    nkb = -(-Sk // FA_MASK_BLOCK_K)
    if block_mask.dim() != 4 or tuple(block_mask.shape[2:]) != (nqb, nkb):
        raise ValueError(f"block_mask must be [1 or B, 1 or HKV or H, {nqb}, {nkb}], "
                         f"got {tuple(block_mask.shape)}")


def fwd_into(q, k, v, o, lse, *, causal=False, window=0, scale=None, num_splits=0, stream=None,
             block_mask=None):
    """Run the forward pass into caller-provided o and lse. Returns (o, lse)."""
    import torch
    _check(q, k, v)
    B, H, Sq, D = q.shape
    HKV, Sk = k.shape[1], k.shape[2]
    if o.shape != q.shape or o.dtype != q.dtype or not o.is_cuda:
        raise ValueError("o must be a device tensor with q's shape and dtype")
    if o.stride(3) != 1 and o.shape[3] > 1:
        raise ValueError("o: the head dimension must be contiguous (stride 1)")
    if tuple(lse.shape) != (B, H, Sq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, H, Sq]")
    if scale is None:
        scale = default_scale(D)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    if block_mask is not None:
        if not all(t.is_contiguous() for t in (q, k, v, o)):
            raise ValueError("a block mask needs contiguous q, k, v and o")
        _check_mask(block_mask, B, H, HKV, Sq, Sk, q)
        st = lib().fa_fwd_block_sparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                       lse.data_ptr(), B, H, HKV, Sq, Sk, D,
                                       block_mask.data_ptr(), block_mask.shape[0],
                                       block_mask.shape[1], float(scale), int(bool(causal)),
                                       int(window), _dtype_code(q), int(num_splits),
                                       stream.cuda_stream)
    elif all(t.is_contiguous() for t in (q, k, v, o)):
        st = lib().fa_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                             lse.data_ptr(), B, H, HKV, Sq, Sk, D, float(scale),
                             int(bool(causal)), int(window), _dtype_code(q), int(num_splits),
                             stream.cuda_stream)
    else:
        st3 = [(ctypes.c_longlong * 3)(*t.stride()[:3]) for t in (q, k, v, o)]
        ptr = [ctypes.cast(a, ctypes.c_void_p) for a in st3]
        st = lib().fa_fwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  lse.data_ptr(), B, H, HKV, Sq, Sk, D, *ptr, float(scale),
                                  int(bool(causal)), int(window), _dtype_code(q),
                                  int(num_splits), stream.cuda_stream)
    if st != 0:
        raise FaError(st)
    return o, lse


def fwd_noalloc_into(q, k, v, o, lse, *, causal=False, window=0, scale=None, num_splits=0,
                     stream=None):
    """fwd_into through fa_fwd_noalloc: the library allocates no device memory
    (its key-split partials live in a static per-GPU array). Contiguous
    tensors only. Returns (o, lse)."""
    import torch
    _check(q, k, v)
    B, H, Sq, D = q.shape
    HKV, Sk = k.shape[1], k.shape[2]
    if o.shape != q.shape or o.dtype != q.dtype or not o.is_cuda:
        raise ValueError("o must be a device tensor with q's shape and dtype")
    if tuple(lse.shape) != (B, H, Sq) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, H, Sq]")
    if not all(t.is_contiguous() for t in (q, k, v, o, lse)):
        raise ValueError("fwd_noalloc_into takes contiguous tensors")
    if scale is None:
        scale = default_scale(D)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = lib().fa_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              lse.data_ptr(), B, H, HKV, Sq, Sk, D, float(scale),
                              int(bool(causal)), int(window), _dtype_code(q), int(num_splits),
                              stream.cuda_stream)
    if st != 0:
        raise FaError(st)
    return o, lse


def fwd(q, k, v, *, causal=False, window=0, scale=None, num_splits=0, stream=None,
        block_mask=None):
    """Forward pass; allocates o (with q's memory layout) and lse with torch.
    Returns (o, lse)."""
    import torch
    _check(q, k, v)
    B, H, Sq, _ = q.shape
    with torch.cuda.device(q.device):
        o = torch.empty_like(q)       # keeps q's strides when q is dense
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    return fwd_into(q, k, v, o, lse, causal=causal, window=window, scale=scale,
                    num_splits=num_splits, stream=stream, block_mask=block_mask)


def bwd(q, k, v, o, lse, do, *, causal=False, window=0, scale=None, stream=None,
        block_mask=None):
    """Backward pass: float32 (dq, dk, dv), the gradients of sum(o * do) for
    o, lse = fwd(q, k, v, ...) with the same arguments; o and do have q's
    shape and dtype. Contiguous tensors go through fa_bwd; views with other
    strides (last dimension contiguous, e.g. token-major storage viewed as
    [B, H, S, D]) through fa_bwd_strided, and the gradients then take the
    memory layout of q, k and v. A block mask (as for fwd; contiguous tensors)
    runs fa_bwd_block_sparse."""
    import torch
    _check(q, k, v)
    B, H, Sq, D = q.shape
    HKV, Sk = k.shape[1], k.shape[2]
    for name, t in (("o", o), ("do", do)):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor with q's shape and dtype")
        if t.stride(3) != 1 and t.shape[3] > 1:
            raise ValueError(f"{name}: the head dimension must be contiguous (stride 1)")
    if tuple(lse.shape) != (B, H, Sq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, H, Sq]")
    if scale is None:
        scale = default_scale(D)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    dense = all(t.is_contiguous() for t in (q, k, v, o, do))

    def grad_like(t):
        # a dense view keeps its layout (e.g. token-major); others get contiguous gradients
        if not dense and not t.is_contiguous() and _is_dense_view(t):
            return torch.empty_like(t, dtype=torch.float32)
        return torch.empty(t.shape, dtype=torch.float32, device=t.device)

    with torch.cuda.device(q.device):
        dq, dk, dv = grad_like(q), grad_like(k), grad_like(v)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
            lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, HKV, Sq, Sk, D)
    tail = (float(scale), int(bool(causal)), int(window), _dtype_code(q), stream.cuda_stream)
    if block_mask is not None:
        if not dense:
            raise ValueError("block_mask needs contiguous q, k, v, o, do")
        _check_mask(block_mask, B, H, HKV, Sq, Sk, q)
        st = lib().fa_bwd_block_sparse(*args, block_mask.data_ptr(), block_mask.shape[0],
                                       block_mask.shape[1], *tail)
    elif dense:
        st = lib().fa_bwd(*args, *tail)
    else:
        st3 = [(ctypes.c_longlong * 3)(*t.stride()[:3]) for t in (q, k, v, o, do, dq, dk, dv)]
        ptr = [ctypes.cast(a, ctypes.c_void_p) for a in st3]
        st = lib().fa_bwd_strided(*args, *ptr, *tail)
    if st != 0:
        raise FaError(st)
    return dq, dk, dv


def _is_dense_view(t) -> bool:
    """True when t's elements fill its storage span without gaps or overlap
    (a permutation of a contiguous tensor), so empty_like keeps its layout."""
    span = 1 + sum((n - 1) * s for n, s in zip(t.shape, t.stride()))
    return span == t.numel() and len(set(s for n, s in zip(t.shape, t.stride()) if n > 1)) == \
        sum(1 for n in t.shape if n > 1)


def plan_splits(B, H, HKV, Sq, Sk, D, *, causal=False, window=0, dtype="bf16") -> int:
    """Key-axis split count the library picks for this problem on the current device."""
    code = _dtype_name_code(dtype)
    r = lib().fa_plan_splits(B, H, HKV, Sq, Sk, D, int(bool(causal)), int(window), code)
    if r < 0:
        raise FaError(-r)
    return r


def bwd_plan(B, H, HKV, Sq, Sk, D, num_cus, *, causal=False, window=0, dtype="bf16") -> dict:
    """How the backward pass would run this problem (contiguous tensors, no
    block mask) on a device with num_cus compute units (host only)."""
    code = _dtype_name_code(dtype)
    buf = (ctypes.c_int * 8)()
    r = lib().fa_bwd_plan(B, H, HKV, Sq, Sk, D, int(bool(causal)), int(window), code, num_cus,
                          ctypes.cast(buf, ctypes.c_void_p))
    if r != 0:
        raise FaError(r)
    keys = ("head_dim", "general", "staged", "per_row", "key_chunks", "keys_per_chunk",
            "row_chunks", "rows_per_chunk")
    return dict(zip(keys, list(buf)))


def schedule_table(B, H, HKV, Sq, Sk, D, nslot, *, causal=False, window=0, dtype="f32"):
    """Persistent-launch item lists for nslot workgroups (host only): returns
    (num_splits, offsets[nslot + 1], items)."""
    code = _dtype_name_code(dtype)
    args = (B, H, HKV, Sq, Sk, D, int(bool(causal)), int(window), code, nslot)
    n = lib().fa_schedule_table(*args, None, 0, None)
    if n < 0:
        raise FaError(-n)
    buf = (ctypes.c_int * n)()
    ns = ctypes.c_int(0)
    lib().fa_schedule_table(*args, ctypes.cast(buf, ctypes.c_void_p), n, ctypes.byref(ns))
    table = list(buf)
    return ns.value, table[:nslot + 1], table[nslot + 1:]


def release():
    """Return the split-K workspace pools to the HIP runtime."""
    lib().fa_release()
