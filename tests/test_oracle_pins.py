"""The fp64 oracle against what the definition of attention fixes.

These run on the CPU only.  Each pin is described in oracle_pins.py; this
file adds the pins for the oracle's helpers (bf16 widening, exp2, row
selection).
"""
import numpy as np
import pytest

import oracle
from oracle import brute
import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check(oracle.lib())


def test_bf16_widening_exact():
    # bf16 is the upper half of an IEEE-754 binary32: these values are exact.
    cases = {
        0x3F80: 1.0,
        0xC000: -2.0,
        0x3F81: 1.0 + 2.0 ** -7,
        0x0001: 2.0 ** -133,            # smallest subnormal
        0x7F7F: (2.0 - 2.0 ** -7) * 2.0 ** 127,  # largest finite
        0x8000: -0.0,
        0x4049: 3.140625,
    }
    for bits, val in cases.items():
        got = oracle.bf16_to_f64(bits)
        assert got == val and np.signbit(got) == np.signbit(val), hex(bits)


def test_exp2_matches_50_digit_values():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.uniform(-126, 0, 200), rng.uniform(0, 8, 50),
                        [-126.0, -0.5, 0.0, 1e-7, -1e-7, 7.999]]).astype(np.float32)
    got = oracle.exp2(x)
    for xi, gi in zip(x, got):
        ref = brute.exp2(float(xi))
        assert abs(gi - ref) <= 2.0 * np.spacing(ref), (xi, gi, ref)


def test_exp2_integers_and_limits():
    ints = np.arange(-126, 9, dtype=np.float32)
    assert np.array_equal(oracle.exp2(ints), np.ldexp(1.0, ints.astype(int)))
    assert oracle.exp2(np.array([-np.inf], np.float32))[0] == 0.0


def test_rows_entry_matches_full_dense_and_varlen():
    rng = np.random.default_rng(5)
    # dense bf16 bits
    B, S, H, D = 2, 13, 3, 8
    bits = [rng.integers(0, 1 << 16, (B, S, H, D), dtype=np.uint16) & 0xBFFF for _ in range(3)]
    # keep exponents moderate: clear the top exponent bit (values in +-2^0 .. range)
    bits = [(b & 0x80FF) | 0x3E00 for b in bits]
    for causal in (False, True):
        o_full, l_full = oracle.attention_bf16(*bits, 0.3, causal)
        rows = rng.choice(B * H * S, 20, replace=False)
        o_r, l_r = oracle.attention_rows_bf16(*bits, rows, 0.3, causal)
        for n, r in enumerate(rows):
            b, h, i = r // (H * S), (r // S) % H, r % S
            assert np.array_equal(o_r[n], o_full[b, i, h]), (causal, r)
            assert l_r[n] == l_full[b, h, i]
    # varlen
    cu = np.array([0, 4, 11, 12], np.int32)
    vb = [(rng.integers(0, 1 << 16, (12, H, D), dtype=np.uint16) & 0x80FF) | 0x3E00
          for _ in range(3)]
    o_full, l_full = oracle.attention_bf16(*vb, 0.5, True, cu)
    rows = np.arange(H * 12)
    o_r, l_r = oracle.attention_rows_bf16(*vb, rows, 0.5, True, cu)
    for r in rows:
        h, t = r // 12, r % 12
        assert np.array_equal(o_r[r], o_full[t, h])
        assert l_r[r] == l_full[h, t]


def test_bf16_entry_equals_f64_entry():
    rng = np.random.default_rng(6)
    bits = [(rng.integers(0, 1 << 16, (1, 9, 2, 4), dtype=np.uint16) & 0x80FF) | 0x3E00
            for _ in range(3)]
    vals = [np.vectorize(oracle.bf16_to_f64)(b) for b in bits]
    o1, l1 = oracle.attention_bf16(*bits, 0.4, True)
    o2, l2 = oracle.attention_f64(*vals, 0.4, True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_rejects_bad_shapes():
    z = np.zeros((1, 1, 1, 1))
    with pytest.raises(ValueError):
        oracle.lib().attention_f64(z[:, :0], z[:, :0], z[:, :0], 1.0, False)


def test_rejects_kv_heads_not_dividing_q_heads():
    q = np.zeros((1, 4, 4, 2))
    k = v = np.zeros((1, 4, 3, 2))
    with pytest.raises(ValueError):
        oracle.attention_f64(q, k, v, 0.5, False)


def test_golden_tiny_bruteforce():
    """Stored 50-digit values (tests/golden/tiny_bruteforce.json)."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_bruteforce.json")
    doc = json.load(open(path))
    for c in doc["cases"]:
        o, l = oracle.attention_f64(np.array(c["q"]), np.array(c["k"]), np.array(c["v"]),
                                    c["scale"], c["causal"])
        assert np.max(np.abs(o - np.array(c["o"]))) <= 1e-12
        assert np.max(np.abs(l - np.array(c["lse"]))) <= 1e-12
