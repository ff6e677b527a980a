"""Top-k over logits rows: the sparse-attention indices that consume the
logits.  Test infrastructure (see the package header).

[P2] "FlashMLA" (flash_mla_with_kvcache parameters): `indices` has shape
(batch_size, seq_len_q, topk) and invalid entries are -1; get_mla_metadata
takes `topk` as the sparsity parameter.  The pages do not say how the indices
are chosen beyond "top-k"; this library's definition (compared bit for bit):
  * row i's candidates are the columns j of its range whose logit is not -inf
    (range [clamp(k_start, 0, Skv), clamp(k_end, start, Skv)), or the whole
    row without ranges);
  * they are ranked by value, larger first, -0 below +0, and equal values by
    smaller column, so the first topk are unique;
  * the row's indices are those columns in ascending order, then -1 up to topk.
"""

import numpy as np

from .reference import row_ranges


def topk_indices(logits, topk, k_start=None, k_end=None):
    """int32 [Sq, topk] as defined in the module docstring."""
    logits = np.asarray(logits, dtype=np.float64)
    sq, skv = logits.shape
    if k_start is None:
        s, e = np.zeros(sq, np.int64), np.full(sq, skv, np.int64)
    else:
        s, e = row_ranges(k_start, k_end, skv)
    out = np.full((sq, topk), -1, dtype=np.int32)
    for i in range(sq):
        cols = np.arange(s[i], e[i])
        v = logits[i, s[i]:e[i]]
        keep = ~np.isneginf(v)
        cols, v = cols[keep], v[keep]
        # primary: value descending; then +0 before -0; then column ascending
        order = np.lexsort((cols, np.signbit(v), -v))
        chosen = np.sort(cols[order[:topk]])
        out[i, :chosen.size] = chosen
    return out
