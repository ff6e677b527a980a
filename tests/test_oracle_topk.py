"""Pins for the oracle's top-k selection (CPU only).

Checked against a hand-worked row and against brute force that ranks
candidates by the integer order of their float32 bit patterns (a route that
shares nothing with the oracle's value sort)."""

import struct

import numpy as np
import pytest

import oracle


def _ordered(x):
    """Integer with the order of the float32 total order (-0 below +0)."""
    (b,) = struct.unpack("<I", struct.pack("<f", float(x)))
    return ~b & 0xFFFFFFFF if b & 0x80000000 else b | 0x80000000


def _brute(logits, topk, k_start=None, k_end=None):
    sq, skv = logits.shape
    out = np.full((sq, topk), -1, np.int32)
    for i in range(sq):
        lo, hi = 0, skv
        if k_start is not None:
            lo = min(max(int(k_start[i]), 0), skv)
            hi = min(max(int(k_end[i]), lo), skv)
        cand = [(j, logits[i, j]) for j in range(lo, hi) if not np.isneginf(logits[i, j])]
        cand.sort(key=lambda jv: (-_ordered(jv[1]), jv[0]))
        chosen = sorted(j for j, _ in cand[:topk])
        out[i, :len(chosen)] = chosen
    return out


def test_hand_worked_row():
    row = np.array([[1.0, 3.0, 3.0, -np.inf, 2.0, 0.0, -0.0]], np.float32)
    assert oracle.topk_indices(row, 3).tolist() == [[1, 2, 4]]
    assert oracle.topk_indices(row, 5).tolist() == [[0, 1, 2, 4, 5]]     # +0 before -0
    assert oracle.topk_indices(row, 6).tolist() == [[0, 1, 2, 4, 5, 6]]
    assert oracle.topk_indices(row, 8).tolist() == [[0, 1, 2, 4, 5, 6, -1, -1]]
    assert oracle.topk_indices(row, 2, [2], [7]).tolist() == [[2, 4]]    # range [2, 7)
    assert oracle.topk_indices(row, 2, [5], [5]).tolist() == [[-1, -1]]  # empty range


def test_equal_values_take_the_smallest_columns():
    row = np.full((1, 50), 0.25, np.float32)
    assert oracle.topk_indices(row, 4).tolist() == [[0, 1, 2, 3]]
    assert oracle.topk_indices(row, 4, [10], [40]).tolist() == [[10, 11, 12, 13]]


@pytest.mark.parametrize("seed,sq,skv,topk,ranges", [
    (0, 6, 40, 5, False), (1, 9, 70, 12, True), (2, 4, 33, 40, True), (3, 12, 64, 1, True),
])
def test_matches_brute_force(seed, sq, skv, topk, ranges):
    rng = np.random.default_rng(seed)
    x = np.round(rng.standard_normal((sq, skv)) * 2) / 2          # many ties
    x[rng.random((sq, skv)) < 0.15] = -np.inf
    x[rng.random((sq, skv)) < 0.05] = -0.0
    x = x.astype(np.float32)
    ks = ke = None
    if ranges:
        ks = rng.integers(-5, skv, sq)
        ke = ks + rng.integers(-3, skv, sq)
    got = oracle.topk_indices(x, topk, ks, ke)
    assert np.array_equal(got, _brute(x, topk, ks, ke))
