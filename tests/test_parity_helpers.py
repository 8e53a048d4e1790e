"""The parity gate's own arithmetic (CPU only)."""
import numpy as np
import pytest

from parity import bf16_neighbours, bf16_round, cell_distance, compare


def test_neighbours():
    x = np.array([1.0, -1.0, 3.0, 2.0, 0.0, -2.0])
    lo, hi = bf16_neighbours(x)
    assert np.array_equal(hi[:4], [1.0 + 2 ** -7, -1.0 + 2 ** -8, 3.0 + 2 ** -6, 2.0 + 2 ** -6])
    assert np.array_equal(lo[:4], [1.0 - 2 ** -8, -1.0 - 2 ** -7, 3.0 - 2 ** -6, 2.0 - 2 ** -7])
    assert lo[4] < 0 < hi[4] and lo[5] == -2.0 - 2 ** -6 and hi[5] == -2.0 + 2 ** -7


def test_cell_distance():
    # exact value inside the cell of the GPU value: 0
    assert cell_distance(np.array([3.0]), np.array([3.0 + 2 ** -8]))[0] == 0.0
    # exact value near the midpoint, GPU picked the other neighbour: tiny
    ex = 3.0 + 2 ** -7 + 1e-6          # just above the midpoint of 3 and 3 + 2^-6
    assert bf16_round(np.array([ex]))[0] == 3.0 + 2 ** -6
    assert cell_distance(np.array([3.0]), np.array([ex]))[0] <= 2e-6
    # a genuinely wrong value: distance is the excess beyond half a ulp
    d = cell_distance(np.array([1.0]), np.array([1.1]))[0]
    assert abs(d - (0.1 - 2 ** -8)) < 1e-12


def test_compare_flags_errors():
    ref = np.linspace(-3, 3, 101)
    good = bf16_round(ref)
    st = compare(good, None, ref, None)
    assert st["o_max"] == 0.0
    bad = good.copy()
    bad[7] += 0.05
    assert compare(bad, None, ref, None)["o_max"] > 0.03


def test_gradient_gate_flags_planted_errors():
    """The backward gate passes an exact result, and fails a gradient off by
    more than the derived bound in one element or by a small bias everywhere."""
    from parity import assert_grad_close, compare_grad
    rng = np.random.default_rng(5)
    g = rng.standard_normal(1000)
    mag = np.abs(g) * 4 + 0.5
    assert_grad_close(compare_grad(bf16_round(g), g, mag))
    bad = bf16_round(g).copy()
    bad[17] += 2.0 ** -8 * abs(g[17]) + 2.0 ** -7 * mag[17] + 1e-3
    with pytest.raises(AssertionError):
        assert_grad_close(compare_grad(bad, g, mag))
    with pytest.raises(AssertionError):
        assert_grad_close(compare_grad(g * 1.02, g, mag * 10))
    with pytest.raises(AssertionError):
        assert_grad_close(compare_grad(np.where(np.arange(1000) == 3, np.nan, g), g, mag))
