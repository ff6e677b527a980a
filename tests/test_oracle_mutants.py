"""The oracle's pins must catch plausible mistakes (CPU only).

Each mutant replaces one step of the float64 reference with a plausible wrong
version (the KV scale dropped, the scale taken outside the ReLU, a transposed
operand, an off-by-one range end, a weight sign lost) and the test asserts that
at least one pin fails for it.  Mistakes are planted in the oracle only.
"""

import numpy as np
import pytest

import oracle
from oracle import reference
from tests.test_oracle_reference import (
    test_hand_worked_fp8_example,
    test_oracle_matches_brute_force,
    test_out_of_range_entries_are_exactly_neg_inf_and_ranges_clamp,
    test_pages_zero_problem_check,
)


def _drop_scale(Sdot, w, kvs):
    return _orig(Sdot, w, np.ones_like(kvs))


def _scale_outside_relu(Sdot, w, kvs):
    val, bound = _orig(Sdot, w, np.ones_like(kvs))
    return val * kvs[None, :], bound


def _abs_weights(Sdot, w, kvs):
    return _orig(Sdot, np.abs(w), kvs)


def _no_relu(Sdot, w, kvs):
    x = Sdot * kvs[None, None, :]
    return (w[:, :, None] * x).sum(axis=1), _orig(Sdot, w, kvs)[1]


_orig = reference._weighted_relu_sum


def _ranges_end_inclusive(k_start, k_end, skv):
    s, e = _orig_ranges(k_start, k_end, skv)
    return s, np.minimum(e + 1, skv)


_orig_ranges = reference.row_ranges


def _pins():
    def brute_all():
        for fmt, d in [("fp8", 32), ("mxfp8", 64), ("mxfp4", 64)]:
            test_oracle_matches_brute_force(fmt, d)
    return [test_hand_worked_fp8_example, brute_all,
            test_out_of_range_entries_are_exactly_neg_inf_and_ranges_clamp,
            test_pages_zero_problem_check]


def _some_pin_fails():
    for pin in _pins():
        try:
            pin()
        except AssertionError:
            return True
    return False


@pytest.mark.parametrize("mutant", [_drop_scale, _scale_outside_relu, _abs_weights, _no_relu])
def test_value_mutants_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(reference, "_weighted_relu_sum", mutant)
    assert _some_pin_fails()


def test_range_mutant_is_caught(monkeypatch):
    monkeypatch.setattr(reference, "row_ranges", _ranges_end_inclusive)
    assert _some_pin_fails()


def test_transposed_kv_mutant_is_caught(monkeypatch):
    real = reference._decoded_inputs

    def transposed(fmt, q, q_sf, kv, kv_sf, kv_scale):
        Q, K, kvs = real(fmt, q, q_sf, kv, kv_sf, kv_scale)
        # reverse the head-dim order of KV only: a mis-indexed operand
        return Q, K[:, ::-1].copy(), kvs

    monkeypatch.setattr(reference, "_decoded_inputs", transposed)
    assert _some_pin_fails()


def test_unmutated_oracle_passes_every_pin():
    assert not _some_pin_fails()
    assert oracle.dense_logits is reference.dense_logits
