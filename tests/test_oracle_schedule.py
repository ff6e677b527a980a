"""Pins for the paged work split (CPU only).

The split is checked against an explicit enumeration of the work units: the
flattened (sequence, block) list is cut with integer arithmetic and the first
unit of every piece is read off the list directly.
"""

import numpy as np
import pytest

import oracle


def _explicit(context_lens, block_size, max_ctx, num_splits):
    units = []
    for b, ctx in enumerate(context_lens):
        n = -(-max(0, min(int(ctx), max_ctx)) // block_size)
        units.extend((b, k) for k in range(n))
    w = len(units)
    firsts = []
    for c in range(num_splits + 1):
        u = c * w // num_splits
        firsts.append(units[u] if u < w else (len(context_lens), 0))
    return units, firsts


@pytest.mark.parametrize("ctx,bs,max_ctx,splits", [
    ([1024, 32768, 5000, 1], 64, 32768, 256),
    ([64, 65, 63, 0, 128], 64, 256, 3),
    ([0, 0, 0], 64, 128, 4),
    ([10, 20], 32, 64, 16),
    ([100000, 5], 64, 1024, 7),          # length above max_context_len is cut
    ([1] * 33, 64, 64, 32),
])
def test_schedule_matches_explicit_enumeration(ctx, bs, max_ctx, splits):
    sched = oracle.paged_schedule(np.array(ctx), 4, bs, max_ctx, splits)
    units, firsts = _explicit(ctx, bs, max_ctx, splits)
    assert sched.dtype == np.int32 and sched.shape == (splits + 1, 2)
    assert [tuple(x) for x in sched.tolist()] == firsts


def test_schedule_pieces_cover_every_unit_once_in_order():
    rng = np.random.default_rng(0)
    ctx = rng.integers(1, 3000, 37)
    sched = oracle.paged_schedule(ctx, 2, 64, 4096, 50)
    units, _ = _explicit(ctx, 64, 4096, 50)
    walked = []
    n = -(-np.minimum(ctx, 4096) // 64)
    for c in range(50):
        b, k = sched[c]
        eb, ek = sched[c + 1]
        while (b, k) != (eb, ek):
            walked.append((int(b), int(k)))
            k += 1
            while b < ctx.size and k >= n[b]:
                b, k = b + 1, 0
    assert walked == units
    sizes = np.diff([c * len(units) // 50 for c in range(51)])
    assert sizes.max() - sizes.min() <= 1


# ---------------------------------------------------------------------------
# dense split over 4-row groups
# ---------------------------------------------------------------------------

def _dense_explicit(ks, ke, skv, num_splits):
    """Units by brute force over columns: a group spans the 64-column windows
    from the first to the last one holding a column in any of its rows' ranges
    (one unit if none)."""
    units = []
    for g0 in range(0, len(ks), 4):
        windows = set()
        for r in range(g0, min(g0 + 4, len(ks))):
            for j in range(skv):
                if ks[r] <= j < ke[r]:
                    windows.add(j // 64)
        n = max(windows) - min(windows) + 1 if windows else 1
        units.extend((g0 // 4, k) for k in range(n))
    w = len(units)
    firsts = []
    for c in range(num_splits + 1):
        u = c * w // num_splits
        firsts.append(units[u] if u < w else (-(-len(ks) // 4), 0))
    return units, firsts


@pytest.mark.parametrize("seed,sq,skv,splits", [
    (0, 13, 300, 7),
    (1, 4, 64, 1),
    (2, 33, 1000, 64),
    (3, 9, 129, 200),        # more pieces than units
])
def test_dense_schedule_matches_brute_force(seed, sq, skv, splits):
    rng = np.random.default_rng(seed)
    ks = rng.integers(-30, skv + 30, sq)
    ke = ks + rng.integers(-20, skv, sq)
    ks[0], ke[0] = 5, 5                          # an empty row
    sched = oracle.dense_schedule(ks, ke, skv, splits)
    _, firsts = _dense_explicit(ks, ke, skv, splits)
    assert sched.dtype == np.int32 and sched.shape == (splits + 1, 2)
    assert [tuple(x) for x in sched.tolist()] == firsts


def test_dense_schedule_causal_units_and_empty_groups():
    # rows 0..7 of a causal prefill over 200 columns: row i covers [0, i + 1);
    # groups [0..3] and [4..7] both lie in window 0 -> one unit each.  Rows
    # 8..11 empty -> 1 unit.  Rows 12..15 cover [60, 190) -> windows 0..2.
    ks = np.array([0] * 8 + [50] * 4 + [60] * 4)
    ke = np.array([1, 2, 3, 4, 5, 6, 7, 8] + [50] * 4 + [190] * 4)
    assert oracle.schedule.dense_units(ks, ke, 200).tolist() == [1, 1, 1, 3]
    sched = oracle.dense_schedule(ks, ke, 200, 3)
    assert sched.tolist() == [[0, 0], [2, 0], [3, 1], [4, 0]]
