"""GPU parity of the large MX workload (Sq=8192, Skv=65536, H=64, D=128) in
MXFP8 and MXFP4: the full -inf mask on the device, then 4096 sampled rows
(always rows 0 and Sq-1) compared in full with the oracle.  The 2 GiB output
stays on the device; the sampled rows come back in slices.
"""

import numpy as np
import pytest
import torch

import synth
from tests.gpu_helpers import assert_mask_on_device, assert_rows_close, log, run_dense

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mqa_logits_amd  # noqa: F401


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_mx_8192x65536_4096_full_rows(fmt):
    case = synth.workload_case(4, fmt)
    log(f"[mx] 8192x65536 {fmt}")
    out = run_dense(case)
    torch.cuda.synchronize()
    assert_mask_on_device(out, case.k_start, case.k_end, case.skv, rows_per_chunk=64)
    rows = synth.sampled_rows(case.seed, case.sq, 4096)
    got = out[torch.from_numpy(rows).cuda()].cpu().numpy()       # 1 GiB of fp32
    del out
    torch.cuda.empty_cache()
    assert_rows_close(got, case, rows, f"c4_{fmt}", row_block=2)
