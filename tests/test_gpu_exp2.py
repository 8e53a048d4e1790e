"""The device exp2 polynomial, exhaustively over every float in [-126, 0].

fa_exp2_emu runs the kernel's own polynomial on the GPU; each result,
rounded to bf16, must lie within 2 bf16 ulp of the oracle's fp64 2^x (the
spec bound).  Also checked: x in (0, 8] (a stale running maximum
gives such arguments), and inputs below -127 give exactly +0.
"""
import sys

import numpy as np
import pytest
import torch

import exact_attention_forward_04_amd as fa
import oracle

pytestmark = pytest.mark.gpu


def bf16_of_f32(y: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 (ties to even) as float64, with integer ops (finite y)."""
    b = y.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def ulp_bf16(ref: np.ndarray) -> np.ndarray:
    """bf16 spacing at a positive normal float64: 2^(exponent - 7)."""
    e = (ref.view(np.int64) >> 52) & 0x7FF
    return ((e - 7) << 52).view(np.float64)


def check_bits(lo_bits, hi_bits, chunk=1 << 25):
    """Every float whose bit pattern is in [lo_bits, hi_bits] (same sign)."""
    worst = 0.0
    for start in range(lo_bits, hi_bits + 1, chunk):
        n = min(chunk, hi_bits + 1 - start)
        bits = torch.arange(start, start + n, dtype=torch.int64, device="cuda").to(torch.int32)
        x = bits.view(torch.float32)
        y = fa.exp2_emu(x)
        xh = x.cpu().numpy()
        yh = y.cpu().numpy()
        ref = oracle.exp2(xh)
        err = np.abs(bf16_of_f32(yh) - ref) / ulp_bf16(ref)
        worst = max(worst, float(err.max()))
        assert err.max() <= 2.0, (start, float(err.max()))
    return worst


@pytest.mark.timeout(900)
def test_exhaustive_negative_range():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # negative floats from -0.0 (0x80000000) up to -126.0 (0xC2FC0000)
    lo, hi = 0x80000000, 0xC2FC0000
    # int32 view: bit patterns with the sign bit set are negative ints
    worst = check_bits(lo - (1 << 32), hi - (1 << 32))
    print("[gpu-case] exp2 poly worst error over [-126, 0]: %.3f bf16 ulp" % worst, flush=True)
    # positive side the kernel can see: (0, 8]
    worst_pos = check_bits(0x00000001, 0x41000000)
    print("[gpu-case] exp2 poly worst error over (0, 8]: %.3f bf16 ulp" % worst_pos, flush=True)


def test_tiny_negative_inputs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    x = torch.tensor([-1e-10, -1e-30, -1.4e-45, -6e-8, -0.0], device="cuda")
    y = fa.exp2_emu(x).cpu().numpy()
    ref = oracle.exp2(x.cpu().numpy())
    assert np.all(np.abs(bf16_of_f32(y) - ref) / ulp_bf16(ref) <= 2.0), y


def test_clamp_gives_zero():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    x = torch.tensor([-float("inf"), -127.0, -500.0, -1e30], device="cuda")
    assert torch.all(fa.exp2_emu(x) == 0)
