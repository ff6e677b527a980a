"""GPU parity of the large MX workload (Sq=8192, Skv=65536, H=64, D=128) in
MXFP8 and MXFP4: full -inf mask on the device, complete sampled rows, and
4096 sampled rows at sampled columns (the oracle computes those entries one by
one).  The 2 GiB output stays on the device.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_helpers import assert_close, assert_mask_on_device, log, run_dense

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mqa_logits_amd  # noqa: F401


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_config4_mx_large(fmt):
    case = synth.config_case(4, fmt)
    log(f"[mx] config 4 {fmt}")
    out = run_dense(case)
    torch.cuda.synchronize()
    assert_mask_on_device(out, case.k_start, case.k_end, case.skv, rows_per_chunk=64)
    rows = synth.sampled_rows(case.seed, case.sq, 8)
    ref, bound = oracle.dense_logits(*case.args(), rows=rows, row_block=2)
    assert_close(out[torch.from_numpy(rows).cuda()].cpu().numpy(), ref, bound, f"c4_{fmt}_rows")
    srows = synth.sampled_rows(case.seed, case.sq, 4096)
    rng = np.random.default_rng(case.seed)
    r = np.repeat(srows, 4)
    c = rng.integers(0, case.skv, r.size)
    c[::4] = np.maximum(0, case.k_end[srows] - 1)
    v, b = oracle.dense_entries(*case.args(), r, c)
    got = out[torch.from_numpy(r).cuda(), torch.from_numpy(c).cuda()].cpu().numpy()
    assert_close(got, v, b, f"c4_{fmt}_entries")
    del out
    torch.cuda.empty_cache()
