"""The device exp2 polynomial's coefficients, checked on the CPU.

The coefficients in csrc/exp2_poly.h (this project's Remez fit) are
evaluated here with the same float32 steps the device function takes
(clamp, Cody-Waite split x = n + f, Horner with FMA, exponent add), and the
result is compared with the oracle's fp64 2^x after rounding to bf16: the
requirement is at most 2 bf16 ulp over [-126, 0] (the kernel also sees
x in (0, tau] from a stale maximum).  The exhaustive check of every float in
that range runs on the GPU through fa_exp2_emu.
"""
import os
import re

import numpy as np

import oracle
from parity import bf16_round

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "exact_attention_forward_04_amd", "csrc", "exp2_poly.h")


def coeffs():
    txt = open(HDR).read()
    c = {}
    for k in range(4):
        m = re.search(r"#define FA_EXP2_C%d (\S+)f" % k, txt)
        c[k] = np.float32(float.fromhex(m.group(1)))
    return [c[0], c[1], c[2], c[3]]


def fma32(a, b, c):
    # a*b of two float32 is exact in float64; one rounding for the add, then to float32
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(np.float32)


def device_model(x):
    c = coeffs()
    x = np.maximum(x.astype(np.float32), np.float32(-127.0))
    n = np.floor(x).astype(np.float32)
    f = (x - n).astype(np.float32)       # in [0, 1]; exactly 1 only for tiny negative x
    p = fma32(np.full_like(f, c[3]), f, np.full_like(f, c[2]))
    p = fma32(p, f, np.full_like(f, c[1]))
    p = fma32(p, f, np.full_like(f, c[0]))
    bits = p.view(np.int32) + (n.astype(np.int32) << 23)
    return bits.view(np.float32)


def ulp_bf16(ref):
    # spacing of bf16 at |ref|: 2^(floor(log2|ref|) - 7)
    return np.ldexp(1.0, np.frexp(ref)[1] - 8)


def test_constant_term_is_one():
    assert coeffs()[0] == np.float32(1.0)


def test_within_two_bf16_ulp_dense_sample():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.uniform(-126, 0, 2_000_000), rng.uniform(0, 8, 200_000),
                        np.arange(-126, 9, dtype=np.float64)]).astype(np.float32)
    ref = oracle.exp2(x)
    y = device_model(x).astype(np.float64)
    err = np.abs(bf16_round(y) - ref) / ulp_bf16(ref)
    assert err.max() <= 2.0, err.max()
    # integers are exact powers of two
    ints = np.arange(-126, 9, dtype=np.float32)
    assert np.array_equal(device_model(ints).astype(np.float64), np.ldexp(1.0, ints.astype(int)))


def test_tiny_negative_and_subnormal_inputs():
    # x just below zero: floor(x) = -1 and x - floor(x) rounds to 1.0; the
    # result must still be ~1 (a clamped fraction would give ~2 instead)
    x = np.array([-1e-10, -1e-30, -1.4e-45, -6e-8, -0.0, 1e-30, 1.4e-45], np.float32)
    ref = oracle.exp2(x)
    y = device_model(x).astype(np.float64)
    err = np.abs(bf16_round(y) - ref) / ulp_bf16(ref)
    assert err.max() <= 2.0, err


def test_clamped_inputs_give_zero():
    y = device_model(np.array([-np.inf, -127.0, -200.0, -1e30], np.float32))
    assert np.all(y == 0.0)
