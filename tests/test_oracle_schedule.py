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
