"""The comparison helpers themselves, on the CPU: a few wrong rows that the
global max-abs / rel-L2 figures cannot see must fail the row-by-row check."""
import numpy as np
import pytest

from tests.parity import assert_attention, assert_lse, worst_row


def _outputs(rows=4096, heads=8, d=128, seed=0):
    rng = np.random.default_rng(seed)
    ref = rng.standard_normal((rows, heads, d)) * 2e-3      # |O| of near-flat softmax rows
    got = ref * (1 + rng.standard_normal(ref.shape) * 1e-3)  # ~bf16-sized noise
    return got, ref


def test_one_wrong_row_fails_only_the_row_check():
    got, ref = _outputs()
    got[1234, 5] = 1.1 * ref[1234, 5]  # one (query, head) row 10 % off
    d = got - ref
    assert np.max(np.abs(d)) <= 2e-2 and np.linalg.norm(d) / np.linalg.norm(ref) <= 5e-3  # global figures pass
    wr, r = worst_row(got, ref)
    assert r == 1234 * 8 + 5 and wr > 0.09
    with pytest.raises(AssertionError, match="worst row"):
        assert_attention("bf16", got, ref)


def test_zero_rows_must_be_exact():
    got, ref = _outputs(rows=64)
    ref[3] = 0.0
    got[3] = 0.0
    assert_attention("bf16", got, ref)
    got[3, 0, 0] = 1e-9
    with pytest.raises(AssertionError, match="worst row"):
        assert_attention("bf16", got, ref)


def test_lse_minus_inf_pattern():
    a = np.array([0.5, -np.inf, 2.0])
    assert_lse("f32", a + 1e-6, a)
    with pytest.raises(AssertionError, match="pattern"):
        assert_lse("f32", np.array([0.5, 3.0, 2.0]), a)
