"""CPU oracle for weighted multi-query-attention logits (test infrastructure).

This package is test infrastructure, not part of the product.  Only the test
suite, the smoke check in ``__graft_entry__`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  It shares no code, tables or helpers with the HIP
path under ``mqa_logits_amd/``, and the HIP path never imports it.

What it computes, in float64, straight from the definition:

    logits[i, j] = sum_h w[i, h] * ReLU(kv_scale[j] * <q[i, h, :], kv[j, :]>)
                   for k_start[i] <= j < k_end[i], and -inf elsewhere.

Sources (page titles; sections named where they are cited):
  [P1] "How to Implement MQA (Multi-Query Attention) Logits Computation with
       DeepGEMM" (instagit article).
  [P2] "FlashMLA" (Algolia docs mirror): the sparse `indices` consumer.
  [P3] "[PR #314] fix: SM90 paged MQA logits IMA on next_n=4" (DeepGEMM PR
       mirror).
  [P4] "[PR #435] Improve SM100 MX MQA logits clean-output performance"
       (DeepGEMM PR mirror).

Modules:
  codecs     exact decode of e4m3fn, e2m1 and e8m0 codes (format definitions).
  reference  dense, compressed and paged logits plus the per-entry error bound.
  schedule   the paged and dense work splits the metadata entry points produce.
  topk       the top-k column indices of logits rows.
  brute      exact rational (fractions.Fraction) evaluation for tiny inputs.

Every function is pinned by tests under ``tests/`` marked ``not gpu``.
"""

from . import codecs, reference, schedule, brute, topk  # noqa: F401
from .reference import (  # noqa: F401
    row_ranges,
    dense_logits,
    dense_entries,
    compressed_row_offsets,
    compressed_logits,
    paged_row_ranges,
    paged_logits,
    gather_paged_kv,
)
from .schedule import paged_schedule, dense_schedule  # noqa: F401
from .topk import topk_indices  # noqa: F401
