"""GPU parity of the paged decode path and its work-split metadata.

The metadata must equal the oracle's split bit for bit; the logits must match
the oracle element by element.  Unused pool blocks hold NaN codes and NaN
scales (synth poisons them), so a read through a wrong block index cannot
pass.  Different split counts must give bitwise-identical logits (no work
crosses a column, so the schedule cannot change a value).
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_helpers import assert_close, dev, log, paged_on_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mqa_logits_amd  # noqa: F401


def _run(case, num_splits, clean=True, out=None):
    import mqa_logits_amd as mq
    d = paged_on_device(case)
    sched = mq.paged_mqa_logits_metadata(d["context_lens"], case.next_n, case.block_size,
                                         case.max_context_len, num_splits)
    out = mq.paged_mqa_logits(d["fmt"], d["q"], d["q_sf"], d["kv_pool"], d["kv_sf_pool"],
                              d["kv_scale_pool"], d["weights"], d["context_lens"],
                              d["block_table"], sched, case.next_n, case.max_context_len,
                              clean_logits=clean, out=out)
    torch.cuda.synchronize()
    return out, sched


def _check(case, num_splits, what):
    log(f"[paged] {what} batch={case.batch} next_n={case.next_n} bs={case.block_size} "
        f"fmt={case.fmt} splits={num_splits}")
    out, sched = _run(case, num_splits)
    ref_sched = oracle.paged_schedule(case.context_lens, case.next_n, case.block_size,
                                      case.max_context_len, num_splits)
    assert np.array_equal(sched.cpu().numpy(), ref_sched), "schedule differs"
    ref, bound = oracle.paged_logits(*case.args())
    assert_close(out.cpu().numpy(), ref, bound, what)
    return out


@pytest.mark.parametrize("splits", [1, 7, 256, 1024, 5000])
def test_metadata_matches_oracle_split(splits):
    import mqa_logits_amd as mq
    rng = np.random.default_rng(splits)
    ctx = rng.integers(0, 40000, 300).astype(np.int32)
    ctx[:5] = [0, 1, 64, 65, 32768]
    for bs, max_ctx in [(64, 32768), (32, 40000), (16, 1000)]:
        got = mq.paged_mqa_logits_metadata(dev(ctx), 4, bs, max_ctx, splits)
        ref = oracle.paged_schedule(ctx, 4, bs, max_ctx, splits)
        assert np.array_equal(got.cpu().numpy(), ref), f"bs={bs}"


def test_metadata_max_batch():
    import mqa_logits_amd as mq
    ctx = np.random.default_rng(0).integers(1, 5000, 8192).astype(np.int32)
    got = mq.paged_mqa_logits_metadata(dev(ctx), 2, 64, 5000, 1024)
    assert np.array_equal(got.cpu().numpy(), oracle.paged_schedule(ctx, 2, 64, 5000, 1024))


@pytest.mark.parametrize("next_n", [1, 2, 3, 4])
@pytest.mark.parametrize("bs", [16, 32, 64])
def test_paged_small_matrix(next_n, bs):
    case = synth.paged_case(batch=5, next_n=next_n, h=64, d=128, block_size=bs,
                            num_blocks=400, ctx_lo=1, ctx_hi=1500, max_context_len=1600,
                            seed=10 * next_n + bs, context_lens=[1, 700, 1600, 33, 1025])
    _check(case, 37, f"small_n{next_n}_bs{bs}")


@pytest.mark.parametrize("next_n,bs", [(5, 64), (6, 32), (9, 16), (16, 16)])
def test_paged_more_than_four_query_tokens(next_n, bs):
    # next_n > 4: each sequence's rows are walked in groups of 4 (16 is the
    # largest next_n the entry point takes)
    case = synth.paged_case(batch=4, next_n=next_n, h=64, d=128, block_size=bs,
                            num_blocks=500, ctx_lo=1, ctx_hi=1500, max_context_len=1603,
                            seed=100 + next_n, context_lens=[3, 700, 1603, 1025])
    _check(case, 41, f"next_n{next_n}_bs{bs}")


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_paged_mx(fmt):
    case = synth.paged_case(batch=6, next_n=4, h=64, d=128, block_size=64, num_blocks=300,
                            ctx_lo=100, ctx_hi=3000, max_context_len=3072, fmt=fmt, seed=44)
    _check(case, 50, f"paged_{fmt}")


@pytest.mark.parametrize("h,d", [(16, 64), (32, 128), (8, 64)])
def test_paged_head_dim(h, d):
    case = synth.paged_case(batch=4, next_n=2, h=h, d=d, block_size=32, num_blocks=200,
                            ctx_lo=10, ctx_hi=2000, max_context_len=2048, seed=h + d)
    _check(case, 16, f"paged_h{h}_d{d}")


@pytest.mark.parametrize("splits", [1, 3000])
def test_paged_edge_lengths_and_idle_workers(splits):
    # empty, shorter-than-next_n and longer-than-max_context_len sequences, a
    # width that is not a multiple of 4; one worker for everything, or far
    # more workers than blocks (most walk nothing and only write -inf)
    case = synth.paged_case(batch=6, next_n=4, h=64, d=128, block_size=64, num_blocks=200,
                            ctx_lo=1, ctx_hi=10, max_context_len=1030, seed=61,
                            context_lens=[0, 2, 1030, 5000, 64, 65])
    _check(case, splits, f"paged_edges_s{splits}")


def test_paged_negative_scales_and_keep_mode():
    case = synth.paged_case(batch=3, next_n=4, h=64, d=128, block_size=64, num_blocks=100,
                            ctx_lo=100, ctx_hi=1000, max_context_len=1024, seed=5,
                            poison_unused=False)
    case.kv_scale_pool[::2] *= -1.0
    _check(case, 9, "paged_negative_scales")
    sentinel = 9.5
    out = torch.full((case.batch * case.next_n, case.max_context_len), sentinel,
                     dtype=torch.float32, device="cuda")
    log("[paged] keep mode")
    _run(case, 9, clean=False, out=out)
    got = out.cpu().numpy()
    ref, bound = oracle.paged_logits(*case.args())
    inside = np.isfinite(ref)
    assert np.all(got[~inside] == sentinel)
    assert_close(np.where(inside, got, -np.inf), ref, bound, "paged_keep")


def test_paged_long_contexts():
    # contexts of up to 2^17 tokens (2048 blocks of 64) through a permuted
    # pool, one past max_context_len, one not a whole number of blocks
    case = synth.paged_case(batch=3, next_n=2, h=64, d=128, block_size=64, num_blocks=7000,
                            ctx_lo=0, ctx_hi=0, max_context_len=1 << 17, seed=517,
                            context_lens=[(1 << 17) + 5, 70001, 99999])
    _check(case, 256, "long_contexts")


def test_paged_decode_64x4_full_parity_and_split_independence():
    case = synth.workload_case(3)
    import mqa_logits_amd as mq
    splits = mq.paged_mqa_logits_default_splits(0)
    out = _check(case, splits, "paged_decode")
    log("[paged] decode workload with other split counts")
    for other in (97, 2 * splits):
        out2, _ = _run(case, other)
        assert torch.equal(out.view(torch.int32), out2.view(torch.int32)), f"splits={other}"


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_paged_decode_shape_in_mx_formats_full_parity(fmt):
    # the paged decode workload at full size in the MX formats (the two-wave
    # head split with e8m0 block scales), every row against the oracle
    case = synth.workload_case(3, fmt)
    import mqa_logits_amd as mq
    _check(case, mq.paged_mqa_logits_default_splits(0), f"paged_decode_{fmt}")
