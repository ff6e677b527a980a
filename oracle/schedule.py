"""The work splits that the metadata entry points must produce (paged decode,
and the dense / compressed scheduled path).

Test infrastructure (see the package header).

[P1] "Implementing Paged MQA Logits Computation for Decoding" has a metadata
call, made once per decoding step from the context lengths, the KV block size
and the number of SMs, whose result the paged kernel consumes; [P3] "a97b74d"
(Root cause / Fix) says the metadata is a schedule with one entry per SM plus
one, decoded into (query index, KV block index), and that producer and consumer
must agree on how many query atoms a sequence has.

The split this library defines (integer work, compared bit for bit):
  * sequence b contributes n_b = ceil(min(ctx_b, max_context_len) / block_size)
    work units (b, 0) .. (b, n_b - 1); one unit is one KV block of sequence b
    for all next_n query rows of b (a single query atom);
  * the W = sum_b n_b units, in sequence-major order, are split into
    num_splits contiguous pieces: piece c holds units
    [floor(c * W / num_splits), floor((c + 1) * W / num_splits));
  * schedule[c] = (b, blk) of the first unit of piece c, and
    schedule[num_splits] = (batch, 0).  When W == 0 every entry is (batch, 0).
Because one unit carries all next_n rows, next_n does not change the split; it
is taken so that both sides are called with the same arguments.

The dense split ([P4] "[PR #435] Improve SM100 MX MQA logits clean-output
performance": the reproducer's get_mqa_logits_metadata(starts, ends, ...)
result passed as schedule_meta; Validation: scheduled and unscheduled outputs
are equal) is defined the same way over 4-row groups:
  * group g holds rows 4g .. 4g+3 (those below Sq); with the clamped ranges
    [s_i, e_i), a group whose rows are all empty has 1 unit, otherwise
    ceil((hi - 64 * floor(lo / 64)) / 64) units, lo = min s_i and hi = max e_i
    over its non-empty rows (64-column trips of the union of its ranges);
  * the split and the entries are as above with (g, t) for (b, blk) and
    ceil(Sq / 4) for batch.
"""

import numpy as np


def paged_units(context_lens, block_size, max_context_len):
    ctx = np.minimum(np.asarray(context_lens, dtype=np.int64), max_context_len)
    ctx = np.maximum(ctx, 0)
    return (ctx + block_size - 1) // block_size


def split_units(n, num_splits):
    """int32 [num_splits + 1, 2]: (item, unit) of each piece's first unit for
    items with n[b] units each, as defined in the module docstring."""
    n = np.asarray(n, dtype=np.int64)
    batch = n.size
    prefix = np.zeros(batch + 1, dtype=np.int64)
    np.cumsum(n, out=prefix[1:])
    total = int(prefix[-1])
    out = np.zeros((num_splits + 1, 2), dtype=np.int32)
    for c in range(num_splits + 1):
        u = (c * total) // num_splits
        if u >= total:
            out[c] = (batch, 0)
            continue
        # the unique sequence whose unit interval [prefix[b], prefix[b+1]) holds u
        b = int(np.searchsorted(prefix, u, side="right") - 1)
        out[c] = (b, u - prefix[b])
    return out


def paged_schedule(context_lens, next_n, block_size, max_context_len, num_splits):
    """int32 [num_splits + 1, 2] paged schedule (module docstring)."""
    return split_units(paged_units(context_lens, block_size, max_context_len), num_splits)


def dense_units(k_start, k_end, skv):
    """Units of each 4-row group for the dense split (module docstring)."""
    ks = np.asarray(k_start, dtype=np.int64)
    ke = np.asarray(k_end, dtype=np.int64)
    s = np.clip(ks, 0, skv)
    e = np.clip(ke, s, skv)
    units = []
    for g in range(0, ks.size, 4):
        rows = [r for r in range(g, min(g + 4, ks.size)) if e[r] > s[r]]
        if not rows:
            units.append(1)
            continue
        lo = min(int(s[r]) for r in rows)
        hi = max(int(e[r]) for r in rows)
        start = (lo // 64) * 64
        units.append(-(-(hi - start) // 64))
    return np.array(units, dtype=np.int64)


def dense_schedule(k_start, k_end, skv, num_splits):
    """int32 [num_splits + 1, 2] dense schedule (module docstring)."""
    return split_units(dense_units(k_start, k_end, skv), num_splits)
