"""GPU parity on cancelling dot products, in both precisions.

Inputs (synth.cancelling_*): every aligned group of 8 elements along D holds a
pair of products +-128 c that cancel exactly, so each dot is the sum of small
products 2^-5 .. 2^-2 in size -- products the matrix core's grouped summation
truncates to a 2^-6 or 2^-5 grid.  Every partial sum of these products is
exact in fp32 in any order, so a kernel whose products reach the fp32
accumulation exactly meets the oracle's bound
    |gpu - ref| <= 1e-4 * sum_h |w * kv_scale * <q, kv>| + 1e-6.

  * MQA_PRECISION_EXACT_PRODUCTS must meet that bound, dense, compressed and
    paged, FP8 and MXFP8, H in {32, 64}, D in {64, 128};
  * MQA_PRECISION_DEFAULT must stay inside its documented error class (the
    bound plus default_class_bound), and does NOT meet the literal bound on
    these inputs (a strict xfail records by how much).
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_helpers import (assert_close, dense_class_bound, default_class_bound,
                               dense_on_device, log, paged_on_device)

pytestmark = pytest.mark.gpu

CASES = [(fmt, h, d) for fmt in ("fp8", "mxfp8") for h in (32, 64) for d in (64, 128)]
WIDE = [(fmt, h, d) for fmt in ("mxfp8", "mxfp4") for h in (32, 64) for d in (64, 128)]


def uses_linear_half(h, d):
    """The dense kernels' default precision takes ReLU's linear half on the
    matrix core for H = 64, and for H = 32 with D = 64 (32x32x64 tiles)."""
    return h == 64 or (h == 32 and d == 64)


def _spread_block_scales(rng, sf, octaves=30):
    """Move every e8m0 block scale by up to +-octaves (NaN codes kept)."""
    keep = sf == 0xFF
    moved = np.clip(sf.astype(np.int64) + rng.integers(-octaves, octaves + 1, sf.shape), 90, 164)
    sf[...] = np.where(keep, sf, moved).astype(np.uint8)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mqa_logits_amd  # noqa: F401


def _dense(case, precision, clean=True):
    import mqa_logits_amd as mq
    d = dense_on_device(case)
    out = mq.mqa_logits(d["fmt"], d["q"], d["q_sf"], d["kv"], d["kv_sf"], d["kv_scale"],
                        d["weights"], d["k_start"], d["k_end"], clean_logits=clean,
                        precision=precision)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _ranges(sq, skv):
    ks = np.arange(sq) * 7
    ke = skv - 50 + np.arange(sq)
    return ks, ke


@pytest.mark.parametrize("fmt,h,d", CASES)
def test_exact_products_meet_the_bound_on_cancelling_dots(fmt, h, d):
    sq, skv = 37, 600
    ks, ke = _ranges(sq, skv)
    case = synth.cancelling_dense_case(sq, skv, h, d, fmt, seed=200 + h + d, k_start=ks, k_end=ke)
    log(f"[precision] exact dense {fmt} H={h} D={d}")
    got = _dense(case, "exact")
    ref, bound = oracle.dense_logits(*case.args())
    assert_close(got, ref, bound, f"exact_cancel_{fmt}_h{h}_d{d}")


@pytest.mark.parametrize("fmt,h,d", CASES)
def test_default_precision_stays_in_its_error_class_on_cancelling_dots(fmt, h, d):
    sq, skv = 37, 600
    ks, ke = _ranges(sq, skv)
    case = synth.cancelling_dense_case(sq, skv, h, d, fmt, seed=200 + h + d, k_start=ks, k_end=ke)
    log(f"[precision] default dense {fmt} H={h} D={d}")
    got = _dense(case, "default")
    ref, bound = oracle.dense_logits(*case.args())
    extra = dense_class_bound(case, lin=uses_linear_half(h, d))
    assert_close(got, ref, bound + np.where(np.isfinite(ref), extra, 0.0),
                 f"default_class_cancel_{fmt}_h{h}_d{d}")
    inside = np.isfinite(ref)
    lit = float((np.abs(got[inside] - ref[inside]) / bound[inside]).max())
    log(f"   literal-bound ratio of the default precision: {lit:.3g}")


@pytest.mark.xfail(strict=True, reason=(
    "the default precision truncates products inside each group of 8 (the matrix core's "
    "summation), so cancelling dots exceed the literal bound; measured |gpu-ref|/bound "
    "1.2e3 to 1.6e3 on these inputs (FP8 and MXFP8, H 32 and 64, D 64 and 128)"))
def test_default_precision_misses_the_literal_bound_on_cancelling_dots():
    sq, skv = 37, 600
    ks, ke = _ranges(sq, skv)
    case = synth.cancelling_dense_case(sq, skv, 64, 128, "fp8", seed=392, k_start=ks, k_end=ke)
    got = _dense(case, "default")
    ref, bound = oracle.dense_logits(*case.args())
    assert_close(got, ref, bound, "default_literal_cancel")


@pytest.mark.parametrize("fmt,h,d", [("fp8", 64, 128), ("mxfp8", 32, 64)])
def test_exact_products_compressed_on_cancelling_dots(fmt, h, d):
    import mqa_logits_amd as mq
    sq, skv = 45, 500
    ks, ke = _ranges(sq, skv)
    case = synth.cancelling_dense_case(sq, skv, h, d, fmt, seed=300 + h, k_start=ks, k_end=ke)
    dd = dense_on_device(case)
    log(f"[precision] exact compressed {fmt} H={h} D={d}")
    packed, off = mq.mqa_logits_compressed(dd["fmt"], dd["q"], dd["q_sf"], dd["kv"], dd["kv_sf"],
                                           dd["kv_scale"], dd["weights"], dd["k_start"],
                                           dd["k_end"], precision="exact")
    torch.cuda.synchronize()
    ref, bound, ref_off = oracle.compressed_logits(*case.args())
    assert np.array_equal(off.cpu().numpy(), ref_off)
    assert_close(packed.cpu().numpy(), ref, bound, f"exact_compressed_cancel_{fmt}")


def _paged(case, precision):
    import mqa_logits_amd as mq
    d = paged_on_device(case)
    sched = mq.paged_mqa_logits_metadata(d["context_lens"], case.next_n, case.block_size,
                                         case.max_context_len, 96)
    out = mq.paged_mqa_logits(d["fmt"], d["q"], d["q_sf"], d["kv_pool"], d["kv_sf_pool"],
                              d["kv_scale_pool"], d["weights"], d["context_lens"],
                              d["block_table"], sched, case.next_n, case.max_context_len,
                              precision=precision)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("fmt,h,d", CASES)
def test_paged_on_cancelling_dots_both_precisions(fmt, h, d):
    case = synth.cancelling_paged_case(5, 3, h, d, 32, 300, 60, 900, 1000, fmt, seed=400 + h + d)
    ref, bound = oracle.paged_logits(*case.args())
    log(f"[precision] paged {fmt} H={h} D={d}")
    assert_close(_paged(case, "exact"), ref, bound, f"paged_exact_cancel_{fmt}_h{h}_d{d}")
    # default: the paged kernel evaluates ReLU per head (no linear half)
    extra = np.zeros_like(ref)
    for b in range(case.context_lens.size):
        length = int(min(case.context_lens[b], case.max_context_len))
        kv, kvs = oracle.gather_paged_kv(case.kv_pool, case.kv_scale_pool, case.block_table, b,
                                         length, case.block_size)
        kv_sf = None
        if case.kv_sf_pool is not None:
            kv_sf, _ = oracle.gather_paged_kv(case.kv_sf_pool, None, case.block_table, b, length,
                                              case.block_size)
        r = slice(b * case.next_n, (b + 1) * case.next_n)
        Q = oracle.codecs.decode(fmt, case.q[r], None if case.q_sf is None else case.q_sf[r])
        K = oracle.codecs.decode(fmt, kv, kv_sf)
        s = np.ones(length) if kvs is None else kvs.astype(np.float64)
        extra[r, :length] = default_class_bound(fmt, Q, K, s,
                                                case.weights[r].astype(np.float64), False)
    got = _paged(case, "default")
    assert_close(got, ref, bound + np.where(np.isfinite(ref), extra, 0.0),
                 f"paged_default_class_cancel_{fmt}_h{h}_d{d}")


@pytest.mark.parametrize("fmt", ["fp8", "mxfp8", "mxfp4"])
@pytest.mark.parametrize("h,d", [(32, 128), (64, 128), (64, 64)])
def test_exact_products_on_random_inputs(fmt, h, d):
    sq, skv = 37, 300
    ks = np.arange(sq) * 3
    ke = skv - 40 + np.arange(sq)
    case = synth.dense_case(sq, skv, h, d, fmt, seed=500 + h + d, k_start=ks, k_end=ke)
    log(f"[precision] exact random {fmt} H={h} D={d}")
    got = _dense(case, "exact")
    ref, bound = oracle.dense_logits(*case.args())
    assert_close(got, ref, bound, f"exact_random_{fmt}_h{h}_d{d}")


# Block scales spread over +-30 octaves: a dot is then dominated by its
# largest-scaled blocks and the rest of it sits far below their size, which the
# matrix core's grouped summation (and the linear half's pieces) resolve only
# to the default precision's error class, like the cancelling dots above.

@pytest.mark.parametrize("fmt,h,d", WIDE)
def test_wide_mx_block_scales_both_precisions(fmt, h, d):
    sq, skv = 33, 700
    ks = np.arange(sq) * 5
    ke = skv - 30 + np.arange(sq)
    case = synth.dense_case(sq, skv, h, d, fmt, seed=5100 + h + d, k_start=ks, k_end=ke)
    rng = np.random.default_rng(77 + h + d)
    _spread_block_scales(rng, case.q_sf)
    _spread_block_scales(rng, case.kv_sf)
    ref, bound = oracle.dense_logits(*case.args())
    log(f"[precision] wide block scales {fmt} H={h} D={d}")
    assert_close(_dense(case, "exact"), ref, bound, f"exact_wide_{fmt}_h{h}_d{d}")
    got = _dense(case, "default")
    extra = dense_class_bound(case, lin=uses_linear_half(h, d))
    assert_close(got, ref, bound + np.where(np.isfinite(ref), extra, 0.0),
                 f"default_class_wide_{fmt}_h{h}_d{d}")
    inside = np.isfinite(ref)
    lit = float((np.abs(got[inside] - ref[inside]) / bound[inside]).max())
    log(f"   literal-bound ratio of the default precision: {lit:.3g}")


@pytest.mark.parametrize("fmt,h,d", [("mxfp8", 64, 128), ("mxfp4", 32, 64)])
def test_paged_wide_mx_block_scales_exact_products(fmt, h, d):
    case = synth.paged_case(batch=4, next_n=3, h=h, d=d, block_size=32, num_blocks=200,
                            ctx_lo=50, ctx_hi=900, max_context_len=1000, fmt=fmt, seed=5200 + h)
    rng = np.random.default_rng(88 + h)
    _spread_block_scales(rng, case.q_sf)
    _spread_block_scales(rng, case.kv_sf_pool)
    ref, bound = oracle.paged_logits(*case.args())
    log(f"[precision] paged wide block scales {fmt} H={h} D={d}")
    assert_close(_paged(case, "exact"), ref, bound, f"paged_exact_wide_{fmt}_h{h}_d{d}")
