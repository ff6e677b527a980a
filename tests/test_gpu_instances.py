"""Every kernel instance the library dispatches, on one small ragged problem
each, against the oracle.

The dense path has an instance per (format, heads, head dim, store mode,
logits type, precision) and a scheduled twin of each; the paged path one per
(format, heads, head dim, clean or keep, logits type, precision).  Each test
below takes one (format, heads, head dim) and walks the rest of the matrix,
with fp32 and with bf16 weights (bf16 weights are an input format: the oracle
takes the exact values of the bf16 bits).  Sizes are chosen ragged against
every tiling: 9 rows (4-row groups), 333 columns (16- and 32-token steps,
64- and 128-column trips), an empty row, starts past zero, ends past Skv.

Checks per call: clean logits match the oracle's -inf mask exactly and every
in-range value is within the oracle's bound (bf16 logits: plus the bf16
rounding, 2^-8 (|ref| + bound)); keep mode writes nothing outside the ranges
(a sentinel survives) and matches in range; compressed rows match the packed
oracle; a scheduled call is bit-identical to the unscheduled one.
"""

import itertools

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_helpers import assert_close, dense_on_device, dev, log, paged_on_device

pytestmark = pytest.mark.gpu

FORMATS = ["fp8", "mxfp8", "mxfp4"]
SHAPES = [(8, 64), (8, 128), (16, 64), (16, 128), (32, 64), (32, 128), (64, 64), (64, 128)]
BF16_UNIT = 2.0 ** -8
SENTINEL = 7.25


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mqa_logits_amd  # noqa: F401


def _round_weights_bf16(case):
    """bf16 weights: the case keeps their exact values for the oracle, the
    device gets the bf16 tensor."""
    bits = synth.encode_bf16(case.weights)
    case.weights = synth.decode_bf16(bits).reshape(case.weights.shape)
    return dev(bits.view(np.int16)).view(torch.bfloat16)


def _widen(bound, ref, out_dtype):
    if out_dtype != torch.bfloat16:
        return bound
    fin = np.isfinite(ref)
    return np.where(fin, bound + BF16_UNIT * (np.abs(np.where(fin, ref, 0.0)) + bound), bound)


def _host(t):
    return t.float().cpu().numpy().astype(np.float64)


def _filled(rows, cols, dtype):
    """A sentinel-filled output; bf16 rows get an even stride (the library
    stores bf16 logits in 4-byte pairs)."""
    width = cols + (cols & 1 if dtype == torch.bfloat16 else 0)
    return torch.full((rows, width), SENTINEL, dtype=dtype, device="cuda")[:, :cols]


@pytest.mark.parametrize("h,d", SHAPES)
@pytest.mark.parametrize("fmt", FORMATS)
def test_dense_instances(fmt, h, d):
    import mqa_logits_amd as mq
    sq, skv = 9, 333
    ks = np.array([0, 5, -3, 100, 7, 0, 200, 1, 40])
    ke = np.array([333, 300, 17, 100, 340, 1, 333, 332, 41])      # row 3 empty, row 4 past Skv
    for w_bf16 in (False, True):
        case = synth.dense_case(sq, skv, h, d, fmt, seed=900 + h + d, k_start=ks, k_end=ke)
        dd = dense_on_device(case)
        if w_bf16:
            dd["weights"] = _round_weights_bf16(case)
        ref, bound = oracle.dense_logits(*case.args())
        cref, cbound, coff = oracle.compressed_logits(*case.args())
        sched = mq.mqa_logits_metadata(dd["k_start"], dd["k_end"], skv, 5)
        args = (dd["fmt"], dd["q"], dd["q_sf"], dd["kv"], dd["kv_sf"], dd["kv_scale"],
                dd["weights"], dd["k_start"], dd["k_end"])
        for precision, out_dtype in itertools.product(("default", "exact"),
                                                      (torch.float32, torch.bfloat16)):
            what = f"{fmt}_h{h}_d{d}_w{'bf16' if w_bf16 else 'f32'}_{precision}_{str(out_dtype)[6:]}"
            log(f"[instances] dense {what}")
            kw = dict(logits_dtype=out_dtype, precision=precision)
            b = _widen(bound, ref, out_dtype)
            # clean, unscheduled and scheduled
            clean = mq.mqa_logits(*args, **kw)
            clean_s = mq.mqa_logits(*args, schedule=sched, **kw)
            # keep: the sentinel survives outside the ranges
            keep = _filled(sq, skv, out_dtype)
            keep_s = _filled(sq, skv, out_dtype)
            mq.mqa_logits(*args, clean_logits=False, out=keep, **kw)
            mq.mqa_logits(*args, clean_logits=False, out=keep_s, schedule=sched, **kw)
            # compressed
            packed, off = mq.mqa_logits_compressed(*args, **kw)
            packed_s, _ = mq.mqa_logits_compressed(*args, row_offsets=off, schedule=sched, **kw)
            torch.cuda.synchronize()
            assert torch.equal(clean, clean_s), f"{what}: scheduled clean differs"
            assert torch.equal(keep, keep_s), f"{what}: scheduled keep differs"
            assert torch.equal(packed, packed_s), f"{what}: scheduled compressed differs"
            assert_close(_host(clean), ref, b, f"{what} clean")
            got = _host(keep)
            inside = np.isfinite(ref)
            assert np.all(got[~inside] == SENTINEL), f"{what}: keep mode wrote outside the ranges"
            assert_close(np.where(inside, got, -np.inf), ref, b, f"{what} keep")
            assert np.array_equal(off.cpu().numpy(), coff)
            assert_close(_host(packed), cref, _widen(cbound, cref, out_dtype), f"{what} compressed")


@pytest.mark.parametrize("h,d", SHAPES)
@pytest.mark.parametrize("fmt", FORMATS)
def test_paged_instances(fmt, h, d):
    import mqa_logits_amd as mq
    bs = {8: 16, 16: 32, 32: 64, 64: 16}[h]
    next_n = 5 if h in (8, 32) else 2                      # 5: two 4-row groups, one ragged
    max_ctx = 301
    for w_bf16 in (False, True):
        case = synth.paged_case(batch=3, next_n=next_n, h=h, d=d, block_size=bs, num_blocks=80,
                                ctx_lo=1, ctx_hi=1, max_context_len=max_ctx, fmt=fmt,
                                seed=950 + h + d, context_lens=[3, 301 + 40, 150])
        pd = paged_on_device(case)
        if w_bf16:
            pd["weights"] = _round_weights_bf16(case)
        ref, bound = oracle.paged_logits(*case.args())
        sched = mq.paged_mqa_logits_metadata(pd["context_lens"], next_n, bs, max_ctx, 7)
        args = (fmt, pd["q"], pd["q_sf"], pd["kv_pool"], pd["kv_sf_pool"], pd["kv_scale_pool"],
                pd["weights"], pd["context_lens"], pd["block_table"], sched, next_n, max_ctx)
        rows = case.batch * next_n
        for precision, out_dtype in itertools.product(("default", "exact"),
                                                      (torch.float32, torch.bfloat16)):
            what = f"{fmt}_h{h}_d{d}_w{'bf16' if w_bf16 else 'f32'}_{precision}_{str(out_dtype)[6:]}"
            log(f"[instances] paged {what}")
            kw = dict(logits_dtype=out_dtype, precision=precision)
            b = _widen(bound, ref, out_dtype)
            clean = mq.paged_mqa_logits(*args, **kw)
            keep = _filled(rows, max_ctx, out_dtype)
            mq.paged_mqa_logits(*args, clean_logits=False, out=keep, **kw)
            torch.cuda.synchronize()
            assert_close(_host(clean), ref, b, f"{what} clean")
            got = _host(keep)
            inside = np.isfinite(ref)
            assert np.all(got[~inside] == SENTINEL), f"{what}: keep mode wrote outside the ranges"
            assert_close(np.where(inside, got, -np.inf), ref, b, f"{what} keep")
