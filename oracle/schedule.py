"""The paged work split that the paged metadata entry point must produce.

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
"""

import numpy as np


def paged_units(context_lens, block_size, max_context_len):
    ctx = np.minimum(np.asarray(context_lens, dtype=np.int64), max_context_len)
    ctx = np.maximum(ctx, 0)
    return (ctx + block_size - 1) // block_size


def paged_schedule(context_lens, next_n, block_size, max_context_len, num_splits):
    """int32 [num_splits + 1, 2] schedule as defined in the module docstring."""
    n = paged_units(context_lens, block_size, max_context_len)
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
