"""The num_correct comparison rule of the GPU parity tests, checked on the CPU.

The metric (fused-linear-ce README, "Metrics for free": argmax == target over
valid rows) is compared exactly, except on rows where rounding can flip the
test.  On inputs with planted targets the oracle's count is large and the
allowance tiny, so a kernel that returned 0, or that kept only the first
vocabulary split's argmax, fails the rule.
"""
import numpy as np
import pytest

import oracle
import synth_inputs as si
from gpu_helpers import TOP2_GAP, ambiguous_rows, assert_num_correct


def _planted(n=512, h=128, v=4000, seed=4, **kw):
    inp = si.make_inputs(n, h, v, dtype="bf16", weight_std=0.05, ignore_frac=0.1, seed=seed,
                         plant_frac=0.5, **kw)
    x, w = si.widen(inp["hidden"], "bf16"), si.widen(inp["weight"], "bf16")
    return inp, x, w


def test_planted_inputs_give_a_large_exact_count():
    inp, x, w = _planted()
    fwd = oracle.forward(x, w, None, inp["targets"], reduction="mean")
    assert fwd.num_correct >= 0.3 * fwd.n_valid
    assert ambiguous_rows(fwd).sum() < 0.01 * fwd.num_correct
    assert_num_correct(fwd.num_correct, fwd, min_frac=0.3)


def test_rule_rejects_zero_and_off_by_more_than_the_allowance():
    inp, x, w = _planted()
    fwd = oracle.forward(x, w, None, inp["targets"], reduction="mean")
    amb = int(ambiguous_rows(fwd).sum())
    for bad in (0, fwd.num_correct + amb + 1, fwd.num_correct - amb - 1):
        with pytest.raises(AssertionError):
            assert_num_correct(bad, fwd, min_frac=0.3)


def test_rule_rejects_a_first_split_only_argmax():
    """A merge that kept the first of 8 vocabulary splits' argmax counts only the rows
    whose target lies there: the oracle on that split's weight rows gives that count."""
    inp, x, w = _planted()
    t = inp["targets"]
    fwd = oracle.forward(x, w, None, t, reduction="mean")
    v8 = w.shape[0] // 8
    part = oracle.forward(x, w[:v8], None, np.where(t < v8, t, si.IGNORE_INDEX), reduction="sum")
    with pytest.raises(AssertionError):
        assert_num_correct(part.num_correct, fwd, min_frac=0.3)


def test_ambiguous_rows_definition():
    """Target tied with the maximum -> ambiguous; target the unique maximum, or below the
    maximum by more than the tolerance -> not; ignored rows never."""
    h = 4
    x = np.array([[2.0, 2.0, 0.0, 0.0],            # tie 0/1, target 1
                  [2.0, 0.0, 0.0, 0.0],            # unique max, target 0
                  [2.0, 2.0 - TOP2_GAP / 2, 0, 0],  # near tie, target 2 (far below)
                  [2.0, 2.0, 0.0, 0.0]])           # tie, but ignored
    w = np.eye(h)
    t = np.array([1, 0, 2, si.IGNORE_INDEX], dtype=np.int64)
    fwd = oracle.forward(x, w, None, t, reduction="sum")
    assert list(ambiguous_rows(fwd)) == [True, False, False, False]
