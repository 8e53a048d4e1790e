"""Comparison helpers for GPU-vs-oracle parity (test code, no attention math).

The gate (the benchmark spec): max |dO| <= 1e-2, mean |dO| <= 1e-3 on the bf16
output and max |dLSE| <= 1e-3.  dO is taken against the oracle's fp64 O
rounded once to bf16 (round-to-nearest-even), the best any bf16 output can
be: the exact O alone is already up to half a bf16 ulp (1.6e-2 at |O| = 4)
away from every bf16 value.  The literal fp64 differences are reported too.
"""
from __future__ import annotations

import numpy as np

O_MAX = 1e-2
O_MEAN = 1e-3
LSE_MAX = 1e-3


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even), in one step."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)                  # x = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)   # 8 significant bits


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def tensor_to_f64(t) -> np.ndarray:
    """A torch tensor (any device, bf16 or fp32) as float64 numpy."""
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f64(t.view(torch.int16).numpy().view(np.uint16))
    return t.to(torch.float64).numpy()


def compare(o_gpu, lse_gpu, o_ref, lse_ref):
    """Return a dict of error statistics; o_* are [..., D] float64 arrays."""
    o_gpu = np.asarray(o_gpu, np.float64)
    o_ref = np.asarray(o_ref, np.float64)
    d_bf = np.abs(o_gpu - bf16_round(o_ref))
    d_lit = np.abs(o_gpu - o_ref)
    st = {
        "o_max": float(d_bf.max()) if d_bf.size else 0.0,
        "o_mean": float(d_bf.mean()) if d_bf.size else 0.0,
        "o_max_fp64": float(d_lit.max()) if d_lit.size else 0.0,
        "o_mean_fp64": float(d_lit.mean()) if d_lit.size else 0.0,
        "bf16_floor": float(np.abs(bf16_round(o_ref) - o_ref).max()) if o_ref.size else 0.0,
        "finite": bool(np.all(np.isfinite(o_gpu))),
    }
    if lse_gpu is not None:
        dl = np.abs(np.asarray(lse_gpu, np.float64) - np.asarray(lse_ref, np.float64))
        st["lse_max"] = float(dl.max()) if dl.size else 0.0
        st["finite"] = st["finite"] and bool(np.all(np.isfinite(lse_gpu)))
    return st


def assert_close(st, what=""):
    assert st["finite"], ("non-finite output", what, st)
    assert st["o_max"] <= O_MAX, ("max |dO|", what, st)
    assert st["o_mean"] <= O_MEAN, ("mean |dO|", what, st)
    if "lse_max" in st:
        assert st["lse_max"] <= LSE_MAX, ("max |dLSE|", what, st)
