"""Test infrastructure only: 50-digit brute-force attention for tiny inputs.

An independent second evaluation of the same definition the C oracle writes
out (FlashAttention-4 paper, section 2.1 names multi-head attention; its
formula is the textbook one): every score is formed exactly in rational
arithmetic from the binary input values, then exponentiated at 50 significant
digits *without* subtracting a row maximum, and O_i = sum_j e^{s_ij} v_j /
sum_j e^{s_ij}, LSE_i = ln sum_j e^{s_ij}.  Because it takes a different route
(no max subtraction, no double rounding) it pins the C oracle's two-pass
formulation rather than re-typing it.

Pure-Python loops: only for S <= 16, D <= 8 or so.
"""
from __future__ import annotations

from fractions import Fraction

import mpmath
import numpy as np

DIGITS = 50


def attention(q, k, v, scale, causal, cu_seqlens=None, cu_seqlens_k=None):
    """q: float array [B,Sq,H,D] (dense) or [Tq,H,D] (varlen); k: [B,Sk,Hkv,D] or
    [Tk,Hkv,D], Hkv dividing H (query head h reads K/V head h // (H // Hkv));
    v: k's shape with its own head dimension Dv.  cu_seqlens / cu_seqlens_k:
    varlen query / key offsets (keys default to the query offsets).  Causal
    masking keeps key j for query i when j <= i + Lk - Lq; a row with no key
    gets O = 0 and LSE = -inf.

    Returns (o, lse) as numpy float64 arrays in the oracle's layouts
    (o like q with Dv columns; lse [B,H,Sq] or [H,Tq]).  Inputs must be
    exactly representable binary floats; they are converted exactly to
    fractions.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    mpmath.mp.dps = DIGITS
    sc = Fraction(float(scale))
    if cu_seqlens is None:
        B, Sq, H, D = q.shape
        Sk, Hkv = k.shape[1], k.shape[2]
        qspans = [(b * Sq, Sq) for b in range(B)]
        kspans = [(b * Sk, Sk) for b in range(B)]
        qf = q.reshape(B * Sq, H, D)
        kf = k.reshape(B * Sk, Hkv, D)
        vf = v.reshape(B * Sk, Hkv, v.shape[-1])
        T = B * Sq
    else:
        cq = [int(c) for c in cu_seqlens]
        ck = [int(c) for c in (cu_seqlens_k if cu_seqlens_k is not None else cu_seqlens)]
        B = len(cq) - 1
        qspans = [(cq[b], cq[b + 1] - cq[b]) for b in range(B)]
        kspans = [(ck[b], ck[b + 1] - ck[b]) for b in range(B)]
        qf, kf, vf = q, k, v
        T, H, D = q.shape
        Hkv = k.shape[1]
    group = H // Hkv
    Dv = v.shape[-1]
    o = np.zeros((T, H, Dv), np.float64)
    lse_t = np.zeros((H, T), np.float64)
    for (t0, Lq), (u0, Lk) in zip(qspans, kspans):
        for h in range(H):
            hk = h // group
            for i in range(Lq):
                keys = range(max(0, min(Lk, i + 1 + Lk - Lq))) if causal else range(Lk)
                if len(keys) == 0:
                    lse_t[h, t0 + i] = -np.inf
                    continue
                w = []
                for j in keys:
                    dot = sum(Fraction(float(qf[t0 + i, h, d])) * Fraction(float(kf[u0 + j, hk, d]))
                              for d in range(D))
                    s = sc * dot
                    w.append(mpmath.exp(mpmath.mpf(s.numerator) / s.denominator))
                z = mpmath.fsum(w)
                for d in range(Dv):
                    num = mpmath.fsum(wj * mpmath.mpf(float(vf[u0 + j, hk, d]))
                                      for wj, j in zip(w, keys))
                    o[t0 + i, h, d] = float(num / z)
                lse_t[h, t0 + i] = float(mpmath.log(z))
    if cu_seqlens is None:
        o = o.reshape(B, Sq, H, Dv)
        lse = lse_t.reshape(H, B, Sq).transpose(1, 0, 2).copy()
        return o, lse
    return o, lse_t


def exp2(x: float) -> float:
    """2**x to 50 digits, rounded to the nearest double."""
    mpmath.mp.dps = DIGITS
    return float(mpmath.power(2, mpmath.mpf(float(x))))
