"""GPU parity of dense and compressed weighted MQA logits against the oracle.

Every test runs the HIP path through the C ABI (mqa_logits_amd) on seeded
inputs from synth and compares element by element with oracle/ (see
gpu_helpers for the rules).  Sizes span several 16x16 tiles, several column
chunks and ragged tails; the 2048x32768 prefill workload is checked on every
row and column, after a full mask check on the device.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_helpers import (assert_close, assert_mask_on_device, assert_rows_close,
                               dense_on_device, dev, log, run_dense)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mqa_logits_amd  # noqa: F401  (fails loudly if the library is missing)


def _check_dense(case, clean=True, what=""):
    log(f"[dense] {what or case.name} fmt={case.fmt} Sq={case.sq} Skv={case.skv} "
        f"H={case.h} D={case.d} clean={clean}")
    out = run_dense(case, clean=clean)
    torch.cuda.synchronize()
    ref, bound = oracle.dense_logits(*case.args())
    return assert_close(out.cpu().numpy(), ref, bound, what or case.name, clean=clean)


def test_tiny_256x1024_full_parity():
    _check_dense(synth.workload_case(0))


@pytest.mark.parametrize("fmt", ["fp8", "mxfp8", "mxfp4"])
@pytest.mark.parametrize("h,d", [(8, 64), (16, 128), (32, 64), (64, 128), (64, 64)])
def test_head_and_dim_matrix(fmt, h, d):
    sq, skv = 37, 300
    ks = np.arange(sq) * 3
    ke = skv - 40 + np.arange(sq)
    case = synth.dense_case(sq, skv, h, d, fmt, seed=100 + h + d, k_start=ks, k_end=ke)
    _check_dense(case, what=f"matrix_{fmt}_h{h}_d{d}")


@pytest.mark.parametrize("sq,skv", [(129, 4100), (17, 260), (1, 1), (5, 17), (64, 16)])
def test_unaligned_lengths(sq, skv):
    case = synth.dense_case(sq, skv, 64, 128, "fp8", seed=sq + skv,
                            k_end=np.maximum(0, skv - sq + np.arange(sq) + 1))
    _check_dense(case, what=f"unaligned_{sq}x{skv}")


def test_irregular_windows_nonzero_starts_empty_rows():
    sq, skv = 96, 3000
    rng = np.random.default_rng(7)
    ks = rng.integers(-50, skv + 50, sq)
    ke = ks + rng.integers(-20, 900, sq)
    ks[:4] = [0, 100, 2999, 500]
    ke[:4] = [skv, 100, 3000, 400]          # full, empty, last column, reversed
    case = synth.dense_case(sq, skv, 32, 128, "fp8", seed=8, k_start=ks, k_end=ke)
    _check_dense(case, what="irregular_windows")


def test_all_zero_problem_pages_check():
    # the pages' reproducer check: 0 in range, -inf exactly where col >= end
    for fmt in ["fp8", "mxfp8", "mxfp4"]:
        sq, skv = 64, 1000
        ends = skv - sq + np.arange(sq)
        case = synth.dense_case(sq, skv, 64, 128, fmt, seed=1, k_end=ends, zero=True)
        log(f"[dense] zero problem {fmt}")
        out = run_dense(case).cpu().numpy()
        valid = np.arange(skv)[None, :] < ends[:, None]
        assert np.array_equal(np.isneginf(out), ~valid)
        assert np.all(out[valid] == 0.0)


def test_negative_kv_scales():
    case = synth.dense_case(40, 700, 64, 128, "fp8", seed=12)
    case.kv_scale[::3] *= -1.0
    case.kv_scale[5] = 0.0
    case.kv_scale[6] = -0.0
    _check_dense(case, what="negative_scales")


def test_keep_mode_leaves_out_of_range_untouched():
    sq, skv = 40, 500
    ks = np.arange(sq) * 5
    ke = ks + 200
    case = synth.dense_case(sq, skv, 16, 64, "fp8", seed=4, k_start=ks, k_end=ke)
    sentinel = 12345.5
    out = torch.full((sq, skv), sentinel, dtype=torch.float32, device="cuda")
    log("[dense] keep mode")
    run_dense(case, clean=False, out=out)
    got = out.cpu().numpy()
    ref, bound = oracle.dense_logits(*case.args())
    inside = np.isfinite(ref)
    assert np.all(got[~inside] == sentinel)
    assert_close(np.where(inside, got, -np.inf), ref, bound, "keep", clean=True)


def test_wide_stride_guard_columns_untouched():
    sq, skv, stride = 33, 517, 640
    case = synth.dense_case(sq, skv, 32, 128, "fp8", seed=6, k_end=np.arange(sq) * 15)
    buf = torch.full((sq + 1, stride), 777.0, dtype=torch.float32, device="cuda")
    out = buf[:sq, :skv]
    log("[dense] wide stride + guard rows")
    run_dense(case, out=out)
    b = buf.cpu().numpy()
    assert np.all(b[:sq, skv:] == 777.0) and np.all(b[sq] == 777.0)
    ref, bound = oracle.dense_logits(*case.args())
    assert_close(b[:sq, :skv], ref, bound, "wide_stride")


def test_bitwise_determinism_20_repeats():
    case = synth.dense_case(64, 5000, 64, 128, "fp8", seed=20, k_end=4000 + np.arange(64) * 10)
    d = dense_on_device(case)
    import mqa_logits_amd as mq
    log("[dense] 20 repeats")
    first = None
    for _ in range(20):
        out = mq.mqa_logits(d["fmt"], d["q"], None, d["kv"], None, d["kv_scale"], d["weights"],
                            d["k_start"], d["k_end"])
        if first is None:
            first = out.clone()
        else:
            assert torch.equal(out.view(torch.int32), first.view(torch.int32))


@pytest.mark.parametrize("fmt", ["fp8", "mxfp8", "mxfp4"])
def test_prefill_2048x32768_every_row(fmt):
    # fp8 is the prefill workload; the MX formats run its shape (two column
    # chunks per row group, where the 8192x65536 workload takes one).  Every row, every column.
    case = synth.workload_case(1, fmt)
    log(f"[dense] prefill 2048x32768, {fmt}, every row")
    out = run_dense(case)
    torch.cuda.synchronize()
    assert_mask_on_device(out, case.k_start, case.k_end, case.skv)
    got = out.cpu().numpy()
    del out
    assert_rows_close(got, case, np.arange(case.sq), f"prefill_{fmt}", row_block=4)


# ---------------------------------------------------------------------------
# compressed layout
# ---------------------------------------------------------------------------

def _check_compressed(case, what):
    import mqa_logits_amd as mq
    d = dense_on_device(case)
    log(f"[compressed] {what} Sq={case.sq} Skv={case.skv} H={case.h} D={case.d} fmt={case.fmt}")
    packed, off = mq.mqa_logits_compressed(d["fmt"], d["q"], d["q_sf"], d["kv"], d["kv_sf"],
                                           d["kv_scale"], d["weights"], d["k_start"], d["k_end"])
    torch.cuda.synchronize()
    ref, bound, ref_off = oracle.compressed_logits(*case.args())
    assert np.array_equal(off.cpu().numpy(), ref_off), "row offsets differ"
    assert packed.numel() == ref.size
    assert_close(packed.cpu().numpy(), ref, bound, what)


@pytest.mark.parametrize("fmt,skv", [("fp8", (1 << 20) + 37), ("mxfp4", (1 << 19) + 37)])
def test_long_key_range_sampled_entries(fmt, skv):
    # keys past 2^19 / 2^20 with a ragged end: the full mask on the device,
    # values on sampled columns of every row (each entry depends only on its
    # key, so the oracle runs on the gathered keys), range ends included
    sq = 8
    ks = np.array([0, 0, 5, 1000, skv // 2, 77, skv - 100, 3], np.int32)
    ke = np.array([skv, skv - 1, skv, skv // 2, skv, 78, skv, skv - 36], np.int32)
    case = synth.dense_case(sq, skv, 64, 128, fmt, seed=4242, k_start=ks, k_end=ke)
    log(f"[dense] long key range {fmt} Skv={skv}")
    out = run_dense(case)
    torch.cuda.synchronize()
    assert_mask_on_device(out, case.k_start, case.k_end, skv)
    s, e = oracle.row_ranges(case.k_start, case.k_end, skv)
    rng = np.random.default_rng(7)
    rows, cols = [], []
    for r in range(sq):
        ends = [s[r], s[r] + 1, e[r] - 2, e[r] - 1]
        c = np.concatenate([rng.integers(s[r], e[r], 512), [x for x in ends if s[r] <= x < e[r]]])
        c = np.unique(c)
        rows.append(np.full(c.size, r))
        cols.append(c)
    rows, cols = np.concatenate(rows), np.concatenate(cols)
    keys, at = np.unique(cols, return_inverse=True)
    sub = lambda a: None if a is None else a[keys]
    ref, bound = oracle.dense_entries(fmt, case.q, case.q_sf, sub(case.kv), sub(case.kv_sf),
                                      sub(case.kv_scale), case.weights,
                                      np.zeros(sq, np.int32), np.full(sq, keys.size, np.int32),
                                      rows, at)
    got = out[torch.from_numpy(rows).to(out.device), torch.from_numpy(cols).to(out.device)]
    assert_close(got.cpu().numpy(), ref, bound, f"long_{fmt}")


def test_compressed_2048x4096_full_parity():
    _check_compressed(synth.workload_case(2), "compressed")


@pytest.mark.parametrize("fmt", ["fp8", "mxfp8", "mxfp4"])
def test_compressed_irregular(fmt):
    sq, skv = 70, 1500
    rng = np.random.default_rng(3)
    ks = rng.integers(-10, skv, sq)
    ke = ks + rng.integers(-5, 700, sq)
    case = synth.dense_case(sq, skv, 64, 128, fmt, seed=30, k_start=ks, k_end=ke)
    _check_compressed(case, f"compressed_irregular_{fmt}")


def test_compressed_guard_band():
    import mqa_logits_amd as mq
    case = synth.dense_case(50, 900, 32, 64, "fp8", seed=9,
                            k_start=np.arange(50) * 7, k_end=np.arange(50) * 7 + 300)
    d = dense_on_device(case)
    off = mq.mqa_logits_compressed_offsets(d["k_start"], d["k_end"], case.skv)
    total = int(off[-1].item())
    buf = torch.full((total + 64,), -3.0, dtype=torch.float32, device="cuda")
    log("[compressed] guard band")
    mq.mqa_logits_compressed(d["fmt"], d["q"], None, d["kv"], None, d["kv_scale"], d["weights"],
                             d["k_start"], d["k_end"], row_offsets=off, out=buf[:total])
    b = buf.cpu().numpy()
    assert np.all(b[total:] == -3.0)
    ref, bound, _ = oracle.compressed_logits(*case.args())
    assert_close(b[:total], ref, bound, "compressed_guard")


@pytest.mark.parametrize("sq", [1, 4095, 4096, 4097, 10000])
def test_compressed_offsets_many_rounds(sq):
    """Row offsets over several 4096-row scan rounds, with ragged, empty,
    reversed and out-of-range ranges: bit-exact against the oracle."""
    import mqa_logits_amd as mq
    skv = 3000
    rng = np.random.default_rng([77, sq])
    ks = rng.integers(-100, skv + 100, size=sq).astype(np.int32)
    ke = (ks + rng.integers(-50, 2000, size=sq)).astype(np.int32)
    log(f"[compressed] offsets Sq={sq} Skv={skv}")
    off = mq.mqa_logits_compressed_offsets(dev(ks), dev(ke), skv)
    torch.cuda.synchronize()
    ref = oracle.compressed_row_offsets(ks, ke, skv)
    assert np.array_equal(off.cpu().numpy(), ref)
