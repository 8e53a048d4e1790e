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


def attention(q, k, v, scale, causal, cu_seqlens=None):
    """q: float array [B,S,H,D] (dense) or [T,H,D] (varlen); k, v the same with
    Hkv heads, Hkv dividing H (query head h reads K/V head h // (H // Hkv));
    v may have its own head dimension Dv.

    Returns (o, lse) as numpy float64 arrays in the oracle's layouts
    (o like q; lse [B,H,S] or [H,T]).  Inputs must be exactly representable
    binary floats; they are converted exactly to fractions.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    mpmath.mp.dps = DIGITS
    sc = Fraction(float(scale))
    if cu_seqlens is None:
        B, S, H, D = q.shape
        spans = [(b * S, S) for b in range(B)]
        Hkv = k.shape[2]
        qf = q.reshape(B * S, H, D)
        kf = k.reshape(B * S, Hkv, D)
        vf = v.reshape(B * S, Hkv, v.shape[-1])
        T = B * S
    else:
        cu = [int(c) for c in cu_seqlens]
        B = len(cu) - 1
        spans = [(cu[b], cu[b + 1] - cu[b]) for b in range(B)]
        qf, kf, vf = q, k, v
        T, H, D = q.shape
        Hkv = k.shape[1]
    group = H // Hkv
    Dv = v.shape[-1]
    o = np.zeros((T, H, Dv), np.float64)
    lse_t = np.zeros((H, T), np.float64)
    for (t0, L) in spans:
        for h in range(H):
            hk = h // group
            for i in range(L):
                keys = range(i + 1) if causal else range(L)
                w = []
                for j in keys:
                    dot = sum(Fraction(float(qf[t0 + i, h, d])) * Fraction(float(kf[t0 + j, hk, d]))
                              for d in range(D))
                    s = sc * dot
                    w.append(mpmath.exp(mpmath.mpf(s.numerator) / s.denominator))
                z = mpmath.fsum(w)
                for d in range(Dv):
                    num = mpmath.fsum(wj * mpmath.mpf(float(vf[t0 + j, hk, d]))
                                      for wj, j in zip(w, keys))
                    o[t0 + i, h, d] = float(num / z)
                lse_t[h, t0 + i] = float(mpmath.log(z))
    if cu_seqlens is None:
        o = o.reshape(B, S, H, Dv)
        lse = lse_t.reshape(H, B, S).transpose(1, 0, 2).copy()
        return o, lse
    return o, lse_t


def exp2(x: float) -> float:
    """2**x to 50 digits, rounded to the nearest double."""
    mpmath.mp.dps = DIGITS
    return float(mpmath.power(2, mpmath.mpf(float(x))))
