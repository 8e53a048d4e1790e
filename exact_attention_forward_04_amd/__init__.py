"""MI355X (gfx950) exact attention: Python binding of libfa_mi355x.so.

Every computation runs in the HIP kernels of the shared library; this module
only marshals arguments (torch is used for device memory and streams).  If
the library is missing or no gfx950 GPU is present, calls raise instead of
falling back to anything else.

    o, lse = attention(q, k, v, causal=True)          # q, k, v: [B,S,H,D] bf16 on cuda
    o, lse = attention(q, k, v, causal=True, cu_seqlens=cu, max_seqlen=S)  # [T,H,D]
    dq, dk, dv = attention_backward(q, k, v, o, lse, do, causal=True)
    o = attention_fn(q, k, v, causal=True)            # autograd: o.backward(...) runs fa_bwd

The C ABI it wraps is declared in include/fa.h.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

from . import build as _build

FA_OK = 0
FA_ERR_INVALID_ARG = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_HIP = -3
FA_ERR_NO_DEVICE = -4
FA_ERR_TOO_LARGE = -5
SPLITKV_SCRATCH_BYTES = 16 << 20   # FA_SPLITKV_SCRATCH_BYTES

LIB_PATH = _build.LIB_PATH
_lib = None


class FaError(RuntimeError):
    """A non-zero fa_status from the library."""

    def __init__(self, fn: str, status: int, msg: str):
        super().__init__("%s failed: %s (%d)" % (fn, msg, status))
        self.status = status


class MfmaRate(ctypes.Structure):
    """Mirror of struct fa_mfma_rate (include/fa.h)."""
    _fields_ = [("workers", ctypes.c_int), ("products", ctypes.c_longlong),
                ("ms", ctypes.c_double), ("tflops", ctypes.c_double),
                ("best_tflops", ctypes.c_double), ("clock_mhz", ctypes.c_double),
                ("cycles_per_product", ctypes.c_double)]


class Tuning(ctypes.Structure):
    """Mirror of struct fa_tuning (include/fa.h)."""
    _fields_ = [("tau", ctypes.c_float), ("exp2_emu", ctypes.c_int),
                ("schedule", ctypes.c_int), ("counters", ctypes.c_void_p),
                ("split_levels", ctypes.c_int)]


def load(path: str = LIB_PATH):
    """Load the shared library (building it first only if nothing is built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        _build.build(path)
    lib = _declare(ctypes.CDLL(path))
    _lib = lib
    return lib


def load_sync_debug(path: str = _build.SYNC_DEBUG_LIB_PATH):
    """The race-check build of the forward and backward (FA_SYNC_DEBUG: every
    wait drains every counter, barriers between the pipeline phases), for
    tests that compare it bit for bit with load()'s library."""
    if not os.path.exists(path):
        _build.build(path, defines=("FA_SYNC_DEBUG",), sources=_build.SYNC_DEBUG_SOURCES)
    return _declare(ctypes.CDLL(path))


def _declare(lib):
    """Argument and result types of the library's entry points."""
    P, I, F, LL = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_longlong
    lib.fa_fwd.argtypes = [P, P, P, P, P, I, I, I, I, F, I, P, P]
    lib.fa_fwd.restype = I
    lib.fa_fwd_ex.argtypes = [P, P, P, P, P, I, I, I, I, F, I, P, P, ctypes.POINTER(Tuning)]
    lib.fa_fwd_ex.restype = I
    lib.fa_fwd_gqa.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, P, P, ctypes.POINTER(Tuning)]
    lib.fa_fwd_gqa.restype = I
    lib.fa_fwd_hd.argtypes = [P, P, P, P, P, I, I, I, I, I, I, F, I, P, P, ctypes.POINTER(Tuning)]
    lib.fa_fwd_hd.restype = I
    lib.fa_fwd_general.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, F, I, P, P, P,
                                   ctypes.POINTER(Tuning)]
    lib.fa_fwd_general.restype = I
    lib.fa_fwd_splitkv.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, F, I, P, P, I, P,
                                   ctypes.c_size_t, P]
    lib.fa_fwd_splitkv.restype = I
    lib.fa_fwd_splitkv_noalloc.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, F, I, P, P, I, P]
    lib.fa_fwd_splitkv_noalloc.restype = I
    lib.fa_splitkv_workspace_size.argtypes = [I, I, I, I, I, I]
    lib.fa_splitkv_workspace_size.restype = ctypes.c_size_t
    lib.fa_splitkv_auto_splits.argtypes = [I, I, I, I, I, ctypes.POINTER(I)]
    lib.fa_splitkv_auto_splits.restype = I
    lib.fa_splitkv_auto_splits_gqa.argtypes = [I, I, I, I, I, I, ctypes.POINTER(I)]
    lib.fa_splitkv_auto_splits_gqa.restype = I
    lib.fa_bwd.argtypes = [P] * 10 + [I, I, I, I, I, F, I, P, P]
    lib.fa_bwd.restype = I
    lib.fa_bwd_general.argtypes = [P] * 10 + [I, I, I, I, I, I, F, I, P, P, P]
    lib.fa_bwd_general.restype = I
    lib.fa_bwd_hd.argtypes = [P] * 10 + [I, I, I, I, I, I, I, F, I, P, P, P]
    lib.fa_bwd_hd.restype = I
    lib.fa_tuning_default.argtypes = []
    lib.fa_tuning_default.restype = Tuning
    lib.fa_exp2_emu.argtypes = [P, P, LL, P]
    lib.fa_exp2_emu.restype = I
    lib.fa_schedule.argtypes = [I, I, I, I, I, P, I, P, I, ctypes.POINTER(I), ctypes.POINTER(I)]
    lib.fa_schedule.restype = I
    lib.fa_schedule_gqa.argtypes = [I, I, I, I, I, I, P, I, P, I, ctypes.POINTER(I),
                                    ctypes.POINTER(I)]
    lib.fa_schedule_gqa.restype = I
    lib.fa_schedule_general.argtypes = [I, I, I, I, I, I, P, P, I, P, I, ctypes.POINTER(I),
                                        ctypes.POINTER(I)]
    lib.fa_schedule_general.restype = I
    lib.fa_num_workers.argtypes = [I, ctypes.POINTER(I)]
    lib.fa_num_workers.restype = I
    lib.fa_device_info.argtypes = [ctypes.POINTER(I), ctypes.POINTER(I)]
    lib.fa_device_info.restype = I
    lib.fa_split_plan.argtypes = [I, I, I, I, I, I, ctypes.POINTER(I)]
    lib.fa_split_plan.restype = I
    lib.fa_schedule_split.argtypes = [I, I, I, I, I, I, P, I, ctypes.POINTER(I), ctypes.POINTER(I)]
    lib.fa_schedule_split.restype = I
    lib.fa_mfma_ceiling.argtypes = [I, I, I, ctypes.POINTER(MfmaRate)]
    lib.fa_mfma_ceiling.restype = I
    lib.fa_status_string.argtypes = [I]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = I
    return lib


def status_string(status: int) -> str:
    return load().fa_status_string(int(status)).decode()


def _check(fn: str, status: int):
    if status != FA_OK:
        raise FaError(fn, status, status_string(status))


def default_tuning() -> Tuning:
    return load().fa_tuning_default()


def _require_buffer(t, name: str, shape, dtype, device) -> None:
    """A caller-supplied output or scratch buffer must be exactly what the
    kernels write through a raw pointer: the expected shape and dtype,
    contiguous, on the inputs' device.  Anything else raises ValueError
    before a launch (a smaller buffer would take out-of-bounds writes)."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError("%s must be %s of shape %s" % (name, dtype, tuple(shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.device != device:
        raise ValueError("%s must be on %s" % (name, device))


def _stream_ptr(stream) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def attention(q, k, v, causal: bool = False, scale: Optional[float] = None,
              cu_seqlens=None, max_seqlen: Optional[int] = None, return_lse: bool = True,
              out=None, lse_out=None, tuning: Optional[Tuning] = None, stream=None,
              cu_seqlens_k=None, max_seqlen_k: Optional[int] = None,
              num_splits: Optional[int] = None, workspace=None):
    """Exact attention forward on the GPU.

    q, k, v: contiguous bf16 CUDA tensors.  Dense: q [B,Sq,H,D], k [B,Sk,H_kv,D],
    v [B,Sk,H_kv,D_v].  Varlen: q [Tq,H,D], k [Tk,H_kv,D], v [Tk,H_kv,D_v] with
    cu_seqlens (query offsets) an int32 CUDA tensor of B+1 entries and
    max_seqlen the longest query length; cu_seqlens_k / max_seqlen_k give the
    key offsets and longest key length when they differ from the queries'.
    H_kv divides H (query head h reads K/V head h // (H // H_kv)); D_v may
    differ from D for the (192, 128) pair.  With causal=True and query and key
    lengths that differ the mask is aligned to the bottom-right corner.
    num_splits > 1 splits every key range over that many workgroups
    (fa_fwd_splitkv, for decode-like batches with few query rows), 0 picks a
    count for the device; workspace (a CUDA uint8 tensor of at least
    splitkv_workspace_size(...) bytes) is allocated when not given, and
    workspace="static" uses the library's fixed device scratch instead
    (fa_fwd_splitkv_noalloc: with out and lse_out given nothing is allocated;
    calls that overlap on one device race).
    Returns (o, lse): o like q with D_v columns (bf16), lse fp32 [B,H,Sq] or
    [H,Tq] (None if return_lse is False).
    """
    import torch
    lib = load()
    if workspace is not None and num_splits is None:
        raise ValueError("workspace is used only with num_splits (split-KV)")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("%s must be a contiguous bf16 CUDA tensor" % name)
    dense = cu_seqlens is None
    if cu_seqlens_k is not None and dense:
        raise ValueError("cu_seqlens_k needs cu_seqlens")
    nd = 4 if dense else 3
    if q.dim() != nd or k.dim() != nd or v.dim() != nd:
        raise ValueError("dense inputs are [B, S, H, D]" if dense else "varlen inputs are [T, H, D]")
    if k.shape[-1] != q.shape[-1] or tuple(v.shape[:-1]) != tuple(k.shape[:-1]) or (
            dense and k.shape[0] != q.shape[0]):
        raise ValueError("k must match q's batch and head dimension, v k's leading shape")
    H, D = q.shape[-2], q.shape[-1]
    H_kv, D_v = k.shape[-2], v.shape[-1]
    if H_kv < 1 or H % H_kv != 0:
        raise ValueError("the K/V head count must divide the query head count")
    if dense:
        B, S = q.shape[0], q.shape[1]
        S_k = k.shape[1]
        lse_shape = (B, H, S)
        cu_ptr = cu_k_ptr = None
    else:
        for name, c in (("cu_seqlens", cu_seqlens), ("cu_seqlens_k", cu_seqlens_k)):
            if c is not None and (c.dtype != torch.int32 or not c.is_cuda or not c.is_contiguous()):
                raise ValueError("%s must be a contiguous int32 CUDA tensor" % name)
        if max_seqlen is None:
            raise ValueError("varlen needs max_seqlen")
        if cu_seqlens_k is None:
            if k.shape[0] != q.shape[0]:
                raise ValueError("different query and key token counts need cu_seqlens_k")
            cu_seqlens_k, max_seqlen_k = cu_seqlens, max_seqlen
        elif max_seqlen_k is None:
            raise ValueError("cu_seqlens_k needs max_seqlen_k")
        B = cu_seqlens.numel() - 1
        if cu_seqlens_k.numel() != B + 1:
            raise ValueError("cu_seqlens and cu_seqlens_k must have the same length")
        S, S_k = int(max_seqlen), int(max_seqlen_k)
        lse_shape = (H, q.shape[0])
        cu_ptr, cu_k_ptr = cu_seqlens.data_ptr(), cu_seqlens_k.data_ptr()
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if num_splits is not None and tuning is not None:
        raise ValueError("num_splits (split-KV) takes no tuning: pass one or the other")
    o_shape = tuple(q.shape[:-1]) + (D_v,)
    for name, t in (("k", k), ("v", v)):
        if t.device != q.device:
            raise ValueError("%s must be on %s" % (name, q.device))
    if out is not None:
        _require_buffer(out, "out", o_shape, torch.bfloat16, q.device)
    o = out if out is not None else torch.empty(o_shape, dtype=q.dtype, device=q.device)
    lse = None
    if return_lse:
        if lse_out is not None:
            _require_buffer(lse_out, "lse_out", lse_shape, torch.float32, q.device)
        lse = lse_out if lse_out is not None else torch.empty(lse_shape, dtype=torch.float32,
                                                              device=q.device)
    sp = _stream_ptr(stream)
    tref = ctypes.byref(tuning) if tuning is not None else None
    lse_ptr = lse.data_ptr() if lse is not None else None
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse_ptr)
    if num_splits is not None:
        splits = int(num_splits)
        if splits == 0:
            n = ctypes.c_int(1)
            _check("fa_splitkv_auto_splits_gqa",
                   lib.fa_splitkv_auto_splits_gqa(B, H, H_kv, S, S_k, D, ctypes.byref(n)))
            splits = n.value
        if isinstance(workspace, str):
            if workspace != "static":
                raise ValueError('workspace must be a tensor, None or "static"')
            rc = lib.fa_fwd_splitkv_noalloc(*ptrs, B, H, H_kv, S, S_k, D, D_v, float(scale),
                                            int(bool(causal)), cu_ptr, cu_k_ptr, splits, sp)
            _check("fa_fwd_splitkv_noalloc", rc)
            return o, lse
        need = lib.fa_splitkv_workspace_size(B, H, S, S_k, D_v, splits)
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        if workspace.numel() * workspace.element_size() < need or not workspace.is_contiguous() \
                or workspace.device != q.device:
            raise ValueError("workspace must be a contiguous buffer of at least %d bytes on %s"
                             % (need, q.device))
        rc = lib.fa_fwd_splitkv(*ptrs, B, H, H_kv, S, S_k, D, D_v, float(scale),
                                int(bool(causal)), cu_ptr, cu_k_ptr, splits,
                                workspace.data_ptr(),
                                workspace.numel() * workspace.element_size(), sp)
        _check("fa_fwd_splitkv", rc)
        return o, lse
    if S_k != S or cu_k_ptr != cu_ptr:
        rc = lib.fa_fwd_general(*ptrs, B, H, H_kv, S, S_k, D, D_v, float(scale),
                                int(bool(causal)), cu_ptr, cu_k_ptr, sp, tref)
        _check("fa_fwd_general", rc)
    elif D_v != D:
        rc = lib.fa_fwd_hd(*ptrs, B, H, H_kv, S, D, D_v, float(scale), int(bool(causal)),
                           cu_ptr, sp, tref)
        _check("fa_fwd_hd", rc)
    elif H_kv != H:
        rc = lib.fa_fwd_gqa(*ptrs, B, H, H_kv, S, D, float(scale), int(bool(causal)), cu_ptr,
                            sp, tref)
        _check("fa_fwd_gqa", rc)
    elif tuning is None:
        rc = lib.fa_fwd(*ptrs, B, H, S, D, float(scale), int(bool(causal)), cu_ptr, sp)
        _check("fa_fwd", rc)
    else:
        rc = lib.fa_fwd_ex(*ptrs, B, H, S, D, float(scale), int(bool(causal)), cu_ptr, sp, tref)
        _check("fa_fwd_ex", rc)
    return o, lse


def attention_backward(q, k, v, o, lse, dout, causal: bool = False,
                       scale: Optional[float] = None, cu_seqlens=None,
                       max_seqlen: Optional[int] = None, dq=None, dk=None, dv=None, delta=None,
                       stream=None, cu_seqlens_k=None, max_seqlen_k: Optional[int] = None):
    """Exact attention backward on the GPU (the fa_bwd_general entry point, or
    fa_bwd_hd when v's head dimension D_v differs from q's D).

    q, k, v, causal, scale, cu_seqlens, max_seqlen, cu_seqlens_k and
    max_seqlen_k as given to attention() (query and key lengths may differ,
    causal masks aligned to the bottom-right corner; (D, D_v) one of (64, 64),
    (128, 128), (256, 256), (192, 128)); o and lse its outputs; dout the
    gradient with respect to o (o's shape, contiguous bf16).  Returns
    (dq, dk, dv) shaped like q, k, v (bf16).  dq/dk/dv/delta may be passed
    in to reuse buffers (delta: fp32 scratch of lse's shape).
    """
    import torch
    lib = load()
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("%s must be a contiguous bf16 CUDA tensor" % name)
    if lse is None or lse.dtype != torch.float32 or not lse.is_cuda or not lse.is_contiguous():
        raise ValueError("lse must be the forward's contiguous fp32 CUDA tensor")
    dense = cu_seqlens is None
    nd = 4 if dense else 3
    if any(t.dim() != nd for t in (q, k, v, o, dout)):
        raise ValueError("dense inputs are [B, S, H, D]" if dense else "varlen inputs are [T, H, D]")
    o_shape = tuple(q.shape[:-1]) + (v.shape[-1],)
    if tuple(k.shape[:-1]) != tuple(v.shape[:-1]) or k.shape[:-3] != q.shape[:-3] or \
            k.shape[-1] != q.shape[-1] or tuple(o.shape) != o_shape or \
            tuple(dout.shape) != o_shape:
        raise ValueError("o and dout must be q's shape with v's head dimension; k, v must share "
                         "their leading shape, and k q's batch and head dimension")
    H, D, H_kv = q.shape[-2], q.shape[-1], k.shape[-2]
    D_v = v.shape[-1]
    if H_kv < 1 or H % H_kv != 0:
        raise ValueError("the K/V head count must divide the query head count")
    if dense:
        if cu_seqlens_k is not None:
            raise ValueError("cu_seqlens_k needs cu_seqlens")
        B, S, S_k = q.shape[0], q.shape[1], k.shape[1]
        lse_shape = (B, H, S)
        cu_ptr = cu_k_ptr = None
    else:
        for name, c in (("cu_seqlens", cu_seqlens), ("cu_seqlens_k", cu_seqlens_k)):
            if c is not None and (c.dtype != torch.int32 or not c.is_cuda or not c.is_contiguous()):
                raise ValueError("%s must be a contiguous int32 CUDA tensor" % name)
        if max_seqlen is None:
            raise ValueError("varlen needs max_seqlen")
        if cu_seqlens_k is None:
            if k.shape[0] != q.shape[0]:
                raise ValueError("different query and key token counts need cu_seqlens_k")
            cu_seqlens_k, max_seqlen_k = cu_seqlens, max_seqlen
        elif max_seqlen_k is None:
            raise ValueError("cu_seqlens_k needs max_seqlen_k")
        B = cu_seqlens.numel() - 1
        if cu_seqlens_k.numel() != B + 1:
            raise ValueError("cu_seqlens and cu_seqlens_k must have the same length")
        S, S_k = int(max_seqlen), int(max_seqlen_k)
        lse_shape = (H, q.shape[0])
        cu_ptr, cu_k_ptr = cu_seqlens.data_ptr(), cu_seqlens_k.data_ptr()
    if tuple(lse.shape) != lse_shape:
        raise ValueError("lse must have shape %s" % (lse_shape,))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq = dq if dq is not None else torch.empty_like(q)
    dk = dk if dk is not None else torch.empty_like(k)
    dv = dv if dv is not None else torch.empty_like(v)
    delta = delta if delta is not None else torch.empty(lse_shape, dtype=torch.float32,
                                                        device=q.device)
    for name, t in (("k", k), ("v", v), ("o", o), ("lse", lse), ("dout", dout)):
        if t.device != q.device:
            raise ValueError("%s must be on %s" % (name, q.device))
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _require_buffer(t, name, ref.shape, torch.bfloat16, q.device)
    _require_buffer(delta, "delta", lse_shape, torch.float32, q.device)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
            lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr())
    if D_v == D:
        rc = lib.fa_bwd_general(*ptrs, B, H, H_kv, S, S_k, D, float(scale), int(bool(causal)),
                                cu_ptr, cu_k_ptr, _stream_ptr(stream))
        _check("fa_bwd_general", rc)
    else:
        rc = lib.fa_bwd_hd(*ptrs, B, H, H_kv, S, S_k, D, D_v, float(scale), int(bool(causal)),
                           cu_ptr, cu_k_ptr, _stream_ptr(stream))
        _check("fa_bwd_hd", rc)
    return dq, dk, dv


def _autograd_function():
    import torch

    class _Attention(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, causal, scale, cu_seqlens, max_seqlen, cu_seqlens_k,
                    max_seqlen_k):
            o, lse = attention(q, k, v, causal=causal, scale=scale, cu_seqlens=cu_seqlens,
                               max_seqlen=max_seqlen, cu_seqlens_k=cu_seqlens_k,
                               max_seqlen_k=max_seqlen_k)
            ctx.save_for_backward(q, k, v, o, lse)
            ctx.cfg = (causal, scale, cu_seqlens, max_seqlen, cu_seqlens_k, max_seqlen_k)
            return o

        @staticmethod
        def backward(ctx, do):
            q, k, v, o, lse = ctx.saved_tensors
            causal, scale, cu_seqlens, max_seqlen, cu_seqlens_k, max_seqlen_k = ctx.cfg
            dq, dk, dv = attention_backward(q, k, v, o, lse, do.contiguous(), causal=causal,
                                            scale=scale, cu_seqlens=cu_seqlens,
                                            max_seqlen=max_seqlen, cu_seqlens_k=cu_seqlens_k,
                                            max_seqlen_k=max_seqlen_k)
            return dq, dk, dv, None, None, None, None, None, None

    return _Attention


_attention_fn = None


def attention_fn(q, k, v, causal: bool = False, scale: Optional[float] = None,
                 cu_seqlens=None, max_seqlen: Optional[int] = None, cu_seqlens_k=None,
                 max_seqlen_k: Optional[int] = None):
    """attention() as a differentiable torch op: returns o, and o.backward()
    computes the input gradients with fa_bwd_general (fa_bwd_hd for the
    (192, 128) head dimensions).  Query and key lengths may differ as in
    attention()."""
    global _attention_fn
    if _attention_fn is None:
        _attention_fn = _autograd_function()
    return _attention_fn.apply(q, k, v, causal, scale, cu_seqlens, max_seqlen, cu_seqlens_k,
                               max_seqlen_k)


def splitkv_workspace_size(B: int, H: int, S_q: int, S_k: int, D_v: int, num_splits: int) -> int:
    """Bytes of workspace fa_fwd_splitkv needs (0 when one split is used)."""
    return load().fa_splitkv_workspace_size(B, H, S_q, S_k, D_v, num_splits)


def exp2_emu(x, stream=None):
    """Device polynomial 2^x (the emulated exponential) on a float32 CUDA tensor."""
    import torch
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 CUDA tensor")
    y = torch.empty_like(x)
    rc = load().fa_exp2_emu(x.data_ptr(), y.data_ptr(), x.numel(), _stream_ptr(stream))
    _check("fa_exp2_emu", rc)
    return y


def schedule(B: int, H: int, S: int, D: int, causal: bool, workers: int,
             cu_seqlens=None, max_rounds: int = 4096, H_kv: Optional[int] = None,
             cu_seqlens_k=None):
    """Host-side persistent tile order: (tiles [workers, rounds] int32, BM).

    Tile code = (seq * H + head) * ceil(S / BM) + mblock, -1 = idle.
    cu_seqlens (optional) is a host sequence of B+1 offsets; H_kv (optional)
    the number of K/V heads for grouped-query attention; cu_seqlens_k
    (optional, with cu_seqlens) key offsets of their own, S then being the
    longest query length.
    """
    import numpy as np
    lib = load()
    tiles = np.full((workers, max_rounds), -2, dtype=np.int32)
    cu = None
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    rounds, bm = ctypes.c_int(0), ctypes.c_int(0)
    cu_ptr = None if cu is None else cu.ctypes.data
    if cu_seqlens_k is not None:
        if cu is None:
            raise ValueError("cu_seqlens_k needs cu_seqlens")
        cuk = np.ascontiguousarray(np.asarray(cu_seqlens_k, dtype=np.int32))
        rc = lib.fa_schedule_general(B, H, H if H_kv is None else H_kv, S, D, int(bool(causal)),
                                     cu_ptr, cuk.ctypes.data, workers, tiles.ctypes.data,
                                     max_rounds, ctypes.byref(rounds), ctypes.byref(bm))
        _check("fa_schedule_general", rc)
        return tiles[:, :rounds.value].copy(), bm.value
    if H_kv is None:
        rc = lib.fa_schedule(B, H, S, D, int(bool(causal)), cu_ptr, workers, tiles.ctypes.data,
                             max_rounds, ctypes.byref(rounds), ctypes.byref(bm))
        _check("fa_schedule", rc)
    else:
        rc = lib.fa_schedule_gqa(B, H, H_kv, S, D, int(bool(causal)), cu_ptr, workers,
                                 tiles.ctypes.data, max_rounds, ctypes.byref(rounds),
                                 ctypes.byref(bm))
        _check("fa_schedule_gqa", rc)
    return tiles[:, :rounds.value].copy(), bm.value


def device_info() -> dict:
    """The current device as the library sees it (fa_device_info): compute
    units and peak shader clock."""
    cus, khz = ctypes.c_int(0), ctypes.c_int(0)
    _check("fa_device_info", load().fa_device_info(ctypes.byref(cus), ctypes.byref(khz)))
    return {"cus": cus.value, "peak_clock_mhz": khz.value / 1000.0}


def split_plan(B: int, H: int, S: int, D: int, workers: int, requested: int = -1) -> int:
    """Split levels a dense causal self-attention launch uses (fa_split_plan;
    requested -1: the library's makespan model decides)."""
    n = ctypes.c_int(0)
    _check("fa_split_plan", load().fa_split_plan(B, H, S, D, workers, requested, ctypes.byref(n)))
    return n.value


def schedule_split(B: int, H: int, S: int, D: int, nsplit: int, workers: int,
                   max_rounds: int = 4096):
    """Host-side persistent order of a dense causal batch with nsplit split
    levels: (items [workers, rounds] int32, BM).  Item code =
    ((seq * H + head) * ceil(S / BM) + mblock) * 3 + part, -1 = none."""
    import numpy as np
    tiles = np.full((workers, max_rounds), -2, dtype=np.int32)
    rounds, bm = ctypes.c_int(0), ctypes.c_int(0)
    _check("fa_schedule_split", load().fa_schedule_split(B, H, S, D, nsplit, workers,
                                                         tiles.ctypes.data, max_rounds,
                                                         ctypes.byref(rounds), ctypes.byref(bm)))
    return tiles[:, :rounds.value].copy(), bm.value


def num_workers(D: int = 128) -> int:
    """Persistent workgroups fa_fwd launches on the current device."""
    n = ctypes.c_int(0)
    _check("fa_num_workers", load().fa_num_workers(D, ctypes.byref(n)))
    return n.value


def mfma_ceiling(mode: int = 0, blocks: int = 8192, reps: int = 5) -> dict:
    """The matrix-unit rate on the D = 128 forward's product sequence alone
    (fa_mfma_ceiling): mode 0 with operands in registers, mode 1 with K and
    V^T read from LDS as the forward reads them.  Synchronous; returns the
    median launch's figures as a dict."""
    r = MfmaRate()
    _check("fa_mfma_ceiling", load().fa_mfma_ceiling(int(mode), int(blocks), int(reps),
                                                     ctypes.byref(r)))
    return {name: getattr(r, name) for name, _ in MfmaRate._fields_}


def version() -> int:
    return load().fa_version()
