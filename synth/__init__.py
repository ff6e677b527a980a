"""Seeded synthetic inputs for weighted MQA logits.

This module only draws random numbers and encodes them into the input formats
(fp8 e4m3fn codes, packed e2m1 codes, e8m0 block scales, fp32 scales, fp32 or
bf16 weights, ranges, paged block tables).  It holds none of the logits
arithmetic.  Both the oracle-side tests and the GPU-side tests and benchmark
take their inputs from here, so the two sides see identical bytes.
"""

from .workloads import (  # noqa: F401
    DenseCase,
    PagedCase,
    encode_bf16,
    decode_bf16,
    encode_e4m3,
    encode_e2m1,
    pack_e2m1,
    dense_case,
    paged_case,
    cancelling_dense_case,
    cancelling_paged_case,
    cancel_pairs,
    CANCEL_BIG,
    workload_case,
    WORKLOAD_NAMES,
    sampled_rows,
    topk_logits,
)
