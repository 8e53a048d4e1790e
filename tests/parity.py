"""Comparison helpers for GPU-vs-oracle parity (test code, no attention math).

The gate: max |dO| <= 1e-2 and mean |dO| <= 1e-3 on the bf16 output, and
max |dLSE| <= 1e-3 on the fp32 log-sum-exp.

Reading of "(bf16 O)": the output is bf16, so even a perfect result is off
the exact value by up to half a bf16 ulp (0.0156 once |O| >= 4), and when the
exact value sits near the midpoint of two bf16 numbers any tiny
pre-rounding error may pick either neighbour.  The max gate therefore
measures the error the kernel adds *before* its one unavoidable output
rounding: dO_i is the distance from the exact O_i to the rounding cell of
the GPU's bf16 value (zero when O_gpu == bf16(O_exact)).  The mean gate and
the reported "o_max_fp64" / "o_mean_fp64" use the literal |O_gpu - O_exact|.
"""
from __future__ import annotations

import os

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


def bf16_neighbours(x: np.ndarray):
    """(next bf16 below, next bf16 above) of bf16-representable float64 values."""
    x = np.asarray(x, np.float64)
    bits = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.int64)
    mag, neg = bits & 0x7FFF, (bits & 0x8000) != 0

    def val(sign, m):
        b = ((sign.astype(np.int64) << 15) | m).astype(np.uint32) << 16
        return b.view(np.float32).astype(np.float64)
    away = val(neg, np.minimum(mag + 1, 0x7F7F))             # larger magnitude
    toward = np.where(mag == 0, -val(neg, np.ones_like(mag)),  # across zero
                      val(neg, np.maximum(mag - 1, 0)))
    lo = np.where(neg, away, toward)
    hi = np.where(neg, toward, away)
    return lo, hi


def cell_distance(o_gpu: np.ndarray, o_ref: np.ndarray) -> np.ndarray:
    """Distance from o_ref to the set of reals that round (to nearest) to o_gpu."""
    lo, hi = bf16_neighbours(o_gpu)
    c_lo = 0.5 * (lo + o_gpu)
    c_hi = 0.5 * (o_gpu + hi)
    return np.maximum(np.maximum(c_lo - o_ref, o_ref - c_hi), 0.0)


def compare(o_gpu, lse_gpu, o_ref, lse_ref):
    """Return a dict of error statistics; o_* are [..., D] float64 arrays,
    o_gpu holding bf16 values."""
    o_gpu = np.asarray(o_gpu, np.float64)
    o_ref = np.asarray(o_ref, np.float64)
    d_cell = cell_distance(o_gpu, o_ref)
    d_lit = np.abs(o_gpu - o_ref)
    st = {
        "o_max": float(d_cell.max()) if d_cell.size else 0.0,
        "o_mean": float(d_lit.mean()) if d_lit.size else 0.0,
        "o_max_vs_bf16_exact": float(np.abs(o_gpu - bf16_round(o_ref)).max()) if o_ref.size else 0.0,
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


# Figures of every parity check run in this process, in order:
# (test id, case, kind, statistics).  conftest.py prints them at the end of
# the pytest session, so a run's log carries each configuration's errors.
FIGURES = []


def record(kind: str, what: str, st: dict) -> None:
    test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
    FIGURES.append((test, str(what), kind, dict(st)))


def assert_close(st, what=""):
    record("forward", what, st)
    assert st["finite"], ("non-finite output", what, st)
    assert st["o_max"] <= O_MAX, ("max |dO|", what, st)
    assert st["o_mean"] <= O_MEAN, ("mean |dO|", what, st)
    if "lse_max" in st:
        assert st["lse_max"] <= LSE_MAX, ("max |dLSE|", what, st)


# ---- backward (gradients dQ, dK, dV; bf16 outputs)
#
# Gate, derived from the arithmetic: a gradient g is a sum of terms whose
# bf16 operands (P or dS, and O inside Delta = <dO, O>) carry a relative
# rounding error of at most u = 2^-8 each, so its error before the output
# rounding is at most about u * A, with A the sum of the terms' absolute
# values (the oracle returns A next to g); the output rounding adds at most
# u * |g|.  The gate allows twice the operand term, for fp32 accumulation
# and exp2 error:  |g_gpu - g| <= 2^-8 |g| + 2^-7 A  elementwise, and a
# relative RMS error ||g_gpu - g|| / ||g|| <= 1e-2 over the tensor (an
# emulation of the kernel's rounding in fp32 gives 2.3e-3 to 3.2e-3).
GRAD_REL_RMS = 1e-2


def compare_grad(g_gpu, g_ref, mag):
    g_gpu = np.asarray(g_gpu, np.float64)
    g_ref = np.asarray(g_ref, np.float64)
    mag = np.asarray(mag, np.float64)
    err = np.abs(g_gpu - g_ref)
    bound = 2.0 ** -8 * np.abs(g_ref) + 2.0 ** -7 * mag
    nrm = float(np.sqrt((g_ref ** 2).sum()))
    return {
        "max_err": float(err.max()) if err.size else 0.0,
        "bound_use": float((err / np.maximum(bound, 1e-300)).max()) if err.size else 0.0,
        "rel_rms": float(np.sqrt((err ** 2).sum()) / nrm) if nrm > 0 else float(err.max(initial=0.0)),
        "finite": bool(np.all(np.isfinite(g_gpu))),
    }


def assert_grad_close(st, what=""):
    record("gradient", what, st)
    assert st["finite"], ("non-finite gradient", what, st)
    assert st["bound_use"] <= 1.0, ("elementwise gradient bound", what, st)
    assert st["rel_rms"] <= GRAD_REL_RMS, ("relative RMS gradient error", what, st)
