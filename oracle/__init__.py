"""Test infrastructure only: the fp64 CPU oracle for exact attention.

The oracle is a plain, slow, double-precision C implementation of
O = softmax(scale * Q K^T + causal mask) V and the row logsumexp, and of the
gradients of sum <dO, O> with respect to Q, K and V (``attn_oracle.c``),
plus a 50-digit brute-force evaluator for tiny forward inputs
(``brute.py``).  It shares no code with the HIP library and never imports it.
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it; the product path must never route through it.

Every method below is a thin ctypes wrapper; the arithmetic lives in C.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "attn_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")


def build(force: bool = False, src: str = SOURCE, out: str = LIB_PATH) -> str:
    """Compile an oracle C source into a shared library with gcc + OpenMP."""
    stale = not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src)
    if force or stale:
        tmp = out + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC",
               "-std=c11", "-o", tmp, src, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


def _ptr(a):
    return None if a is None else a.ctypes.data


def _as_bits(t) -> np.ndarray:
    """bf16 data as a contiguous uint16 numpy array of its bit patterns.

    Accepts a numpy uint16 array or a CPU torch bfloat16 tensor.
    """
    if isinstance(t, np.ndarray):
        assert t.dtype == np.uint16
        return np.ascontiguousarray(t)
    import torch  # local: torch is only needed when handed a tensor
    assert t.dtype == torch.bfloat16 and t.device.type == "cpu"
    return np.ascontiguousarray(t.contiguous().view(torch.int16).numpy().view(np.uint16))


def _is_bf16(t) -> bool:
    if isinstance(t, np.ndarray):
        return t.dtype == np.uint16
    import torch
    return isinstance(t, torch.Tensor) and t.dtype == torch.bfloat16


def _cu(cu_seqlens):
    if cu_seqlens is None:
        return None
    return np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))


def _maxlen(cu) -> int:
    return int(np.max(np.diff(cu))) if len(cu) > 1 else 0


def _layout(q_shape, k_shape, v_shape, cu_q, cu_k):
    """Sizes (B, H, Hkv, Sq, Sk, D, Dv) of a call.

    dense : q [B,Sq,H,D], k [B,Sk,Hkv,D], v [B,Sk,Hkv,Dv]
    varlen: q [Tq,H,D], k [Tk,Hkv,D], v [Tk,Hkv,Dv]; Sq, Sk the longest lengths
    """
    if cu_q is None:
        B, Sq, H, D = q_shape
        Sk, Hkv = k_shape[1], k_shape[2]
    else:
        _, H, D = q_shape
        Hkv = k_shape[1]
        B = len(cu_q) - 1
        Sq, Sk = _maxlen(cu_q), _maxlen(cu_k)
    return B, H, Hkv, Sq, Sk, D, v_shape[-1]


def _out_shapes(B, H, Sq, Dv, cu_q):
    """Shapes of o (Dv columns) and lse."""
    if cu_q is None:
        return (B, Sq, H, Dv), (B, H, Sq)
    T = int(cu_q[-1])
    return (T, H, Dv), (H, T)


class OracleLib:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
        dims = [i32] * 7  # B, H, Hkv, Sq, Sk, D, Dv
        lib.oracle_attn_fwd_f64.argtypes = [P, P, P, P, P] + dims + [f64, i32, P, P]
        lib.oracle_attn_fwd_bf16.argtypes = [P, P, P, P, P] + dims + [f64, i32, P, P]
        lib.oracle_attn_rows_bf16.argtypes = [P, P, P, P, i64, P, P] + dims + [f64, i32, P, P]
        lib.oracle_attn_bwd_f64.argtypes = [P] * 10 + dims + [f64, i32, P, P]
        lib.oracle_attn_bwd_bf16.argtypes = [P] * 10 + dims + [f64, i32, P, P]
        lib.oracle_attn_bwd_rows_bf16.argtypes = ([P, P, P, P, P, i64, P, P, P, i64, P, P, P, P]
                                                  + dims + [f64, i32, P, P])
        for fn in (lib.oracle_attn_fwd_f64, lib.oracle_attn_fwd_bf16, lib.oracle_attn_rows_bf16,
                   lib.oracle_attn_bwd_f64, lib.oracle_attn_bwd_bf16,
                   lib.oracle_attn_bwd_rows_bf16):
            fn.restype = i32
        lib.oracle_exp2.argtypes = [P, P, i64]
        lib.oracle_exp2.restype = None
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = i32
        lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_f64.restype = f64
        self.lib = lib
        self.path = path

    def attention_f64(self, q, k, v, scale, causal, cu_seqlens=None, cu_seqlens_k=None):
        """Attention on float64 inputs.

        q is [B,Sq,H,D] (or [T,H,D] varlen); k has the same layout with Hkv
        heads (Hkv divides H) and its own length; v is k with Dv columns.
        cu_seqlens are the varlen query offsets and cu_seqlens_k the key
        offsets (default: the same).  Causal masking is aligned to the
        bottom-right corner.  Returns (o float64 like q with Dv columns, lse
        float64 [B,H,Sq] or [H,T]).
        """
        q = np.ascontiguousarray(q, dtype=np.float64)
        k = np.ascontiguousarray(k, dtype=np.float64)
        v = np.ascontiguousarray(v, dtype=np.float64)
        return self._run(self.lib.oracle_attn_fwd_f64, q, k, v, scale, causal, cu_seqlens,
                         cu_seqlens_k, "oracle_attn_fwd_f64")

    def attention_bf16(self, q, k, v, scale, causal, cu_seqlens=None, cu_seqlens_k=None):
        """Attention on bf16 inputs (torch bf16 CPU tensors or uint16 bit arrays).

        Shapes as in attention_f64; the result is float64.
        """
        qb, kb, vb = _as_bits(q), _as_bits(k), _as_bits(v)
        return self._run(self.lib.oracle_attn_fwd_bf16, qb, kb, vb, scale, causal, cu_seqlens,
                         cu_seqlens_k, "oracle_attn_fwd_bf16")

    def _run(self, fn, q, k, v, scale, causal, cu_seqlens, cu_seqlens_k, name):
        cu_q = _cu(cu_seqlens)
        cu_k = _cu(cu_seqlens_k) if cu_seqlens_k is not None else cu_q
        B, H, Hkv, Sq, Sk, D, Dv = _layout(q.shape, k.shape, v.shape, cu_q, cu_k)
        o_shape, l_shape = _out_shapes(B, H, Sq, Dv, cu_q)
        o = np.empty(o_shape, np.float64)
        lse = np.empty(l_shape, np.float64)
        rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, Sq, Sk, D, Dv,
                float(scale), int(bool(causal)), _ptr(cu_q), _ptr(cu_k))
        if rc != 0:
            raise ValueError(name + " rejected its arguments")
        return o, lse

    def attention_rows_bf16(self, q, k, v, rows, scale, causal, cu_seqlens=None,
                            cu_seqlens_k=None):
        """Attention for selected rows only.

        rows are numbered like the lse layout: dense (b*H + h)*Sq + i, varlen
        h*Tq + t.  Returns (o_rows float64 [n, Dv], lse_rows float64 [n]).
        """
        qb, kb, vb = _as_bits(q), _as_bits(k), _as_bits(v)
        cu_q = _cu(cu_seqlens)
        cu_k = _cu(cu_seqlens_k) if cu_seqlens_k is not None else cu_q
        B, H, Hkv, Sq, Sk, D, Dv = _layout(qb.shape, kb.shape, vb.shape, cu_q, cu_k)
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        o = np.empty((len(rows), Dv), np.float64)
        lse = np.empty(len(rows), np.float64)
        rc = self.lib.oracle_attn_rows_bf16(_ptr(qb), _ptr(kb), _ptr(vb), _ptr(rows),
                                            len(rows), _ptr(o), _ptr(lse), B, H, Hkv, Sq, Sk,
                                            D, Dv, float(scale), int(bool(causal)),
                                            _ptr(cu_q), _ptr(cu_k))
        if rc != 0:
            raise ValueError("oracle_attn_rows_bf16 rejected its arguments")
        return o, lse

    def attention_backward(self, q, k, v, dout, scale, causal, cu_seqlens=None,
                           cu_seqlens_k=None, magnitudes=False):
        """Gradients of sum <dout, O> with respect to q, k and v.

        Inputs are float64 arrays (any float dtype is widened) or bf16 (torch
        bf16 CPU tensors / uint16 bit arrays, all four alike); dout has o's
        shape (q's with Dv columns).  Returns (dq, dk, dv) as float64 arrays
        shaped like q, k, v; with magnitudes=True also (|dq|, |dk|, |dv|), the
        sums of absolute values of each gradient's terms.
        """
        bf = _is_bf16(q)
        if bf:
            arrs = [_as_bits(t) for t in (q, k, v, dout)]
            fn, name = self.lib.oracle_attn_bwd_bf16, "oracle_attn_bwd_bf16"
        else:
            arrs = [np.ascontiguousarray(t, dtype=np.float64) for t in (q, k, v, dout)]
            fn, name = self.lib.oracle_attn_bwd_f64, "oracle_attn_bwd_f64"
        qa, ka, va, ga = arrs
        cu_q = _cu(cu_seqlens)
        cu_k = _cu(cu_seqlens_k) if cu_seqlens_k is not None else cu_q
        B, H, Hkv, Sq, Sk, D, Dv = _layout(qa.shape, ka.shape, va.shape, cu_q, cu_k)
        o_shape, _ = _out_shapes(B, H, Sq, Dv, cu_q)
        if tuple(ga.shape) != tuple(o_shape):
            raise ValueError("dout must have o's shape %s" % (o_shape,))
        outs = [np.empty(qa.shape), np.empty(ka.shape), np.empty(va.shape)]
        mags = [np.empty(qa.shape), np.empty(ka.shape), np.empty(va.shape)] if magnitudes \
            else [None, None, None]
        rc = fn(_ptr(qa), _ptr(ka), _ptr(va), _ptr(ga), *[_ptr(x) for x in outs],
                *[_ptr(x) for x in mags], B, H, Hkv, Sq, Sk, D, Dv, float(scale),
                int(bool(causal)), _ptr(cu_q), _ptr(cu_k))
        if rc != 0:
            raise ValueError(name + " rejected its arguments")
        return (tuple(outs) + tuple(mags)) if magnitudes else tuple(outs)

    def attention_backward_rows_bf16(self, q, k, v, dout, q_rows, k_rows, scale, causal,
                                     cu_seqlens=None, cu_seqlens_k=None):
        """Backward for selected rows only (bf16 inputs).

        q_rows are numbered like the lse layout (dense (b*H + h)*Sq + i,
        varlen h*Tq + t); k_rows like it over the K/V heads (dense
        (b*Hkv + hk)*Sk + j, varlen hk*Tk + t).  Returns float64
        (dq [nq, D], |dq|, dk [nk, D], dv [nk, Dv], |dk|, |dv|).
        """
        qb, kb, vb, gb = (_as_bits(t) for t in (q, k, v, dout))
        cu_q = _cu(cu_seqlens)
        cu_k = _cu(cu_seqlens_k) if cu_seqlens_k is not None else cu_q
        B, H, Hkv, Sq, Sk, D, Dv = _layout(qb.shape, kb.shape, vb.shape, cu_q, cu_k)
        qr = np.ascontiguousarray(np.asarray(q_rows, dtype=np.int64))
        kr = np.ascontiguousarray(np.asarray(k_rows, dtype=np.int64))
        dq = np.empty((len(qr), D))
        dqm = np.empty((len(qr), D))
        dk = np.empty((len(kr), D))
        dv = np.empty((len(kr), Dv))
        dkm = np.empty((len(kr), D))
        dvm = np.empty((len(kr), Dv))
        rc = self.lib.oracle_attn_bwd_rows_bf16(
            _ptr(qb), _ptr(kb), _ptr(vb), _ptr(gb), _ptr(qr), len(qr), _ptr(dq), _ptr(dqm),
            _ptr(kr), len(kr), _ptr(dk), _ptr(dv), _ptr(dkm), _ptr(dvm), B, H, Hkv, Sq, Sk, D,
            Dv, float(scale), int(bool(causal)), _ptr(cu_q), _ptr(cu_k))
        if rc != 0:
            raise ValueError("oracle_attn_bwd_rows_bf16 rejected its arguments")
        return dq, dqm, dk, dv, dkm, dvm

    def exp2(self, x) -> np.ndarray:
        """2**x in float64 for float32 inputs (what the device polynomial approximates)."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        y = np.empty(x.shape, np.float64)
        self.lib.oracle_exp2(_ptr(x), _ptr(y), x.size)
        return y

    def bf16_to_f64(self, bits: int) -> float:
        """Exact value of one bf16 bit pattern."""
        return self.lib.oracle_bf16_to_f64(int(bits) & 0xFFFF)

    def num_threads(self) -> int:
        """Threads the oracle's OpenMP regions use."""
        return self.lib.oracle_num_threads()


_default = None


def lib() -> OracleLib:
    """The oracle built from attn_oracle.c (compiled on first use)."""
    global _default
    if _default is None:
        _default = OracleLib(build())
    return _default


def attention_f64(*a, **kw):
    return lib().attention_f64(*a, **kw)


def attention_bf16(*a, **kw):
    return lib().attention_bf16(*a, **kw)


def attention_rows_bf16(*a, **kw):
    return lib().attention_rows_bf16(*a, **kw)


def attention_backward(*a, **kw):
    return lib().attention_backward(*a, **kw)


def attention_backward_rows_bf16(*a, **kw):
    return lib().attention_backward_rows_bf16(*a, **kw)


def exp2(x):
    return lib().exp2(x)


def bf16_to_f64(bits):
    return lib().bf16_to_f64(bits)


def num_threads():
    return lib().num_threads()
