"""Seeded random shapes against the oracle: dense, compressed and paged calls
with row counts, key counts, head counts, head dims, formats, logits types,
precisions, ranges, output, block-table and logits row strides and (FP8)
negative or zero token scales drawn per case (small sizes, so the oracle runs in
milliseconds).  Every case checks the oracle's -inf mask and bound, that
guard columns past the row width are never written, and that compressed
offsets match the oracle bit for bit."""

import os

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_helpers import assert_close, dense_on_device, dev, log, paged_on_device

pytestmark = pytest.mark.gpu

BF16_UNIT = 2.0 ** -8
GUARD = -5.5
# more seeds for a longer sweep: MQA_RANDOM_CASES=k multiplies the counts;
# MQA_RANDOM_SIZE=f multiplies the key counts and context lengths drawn
SCALE = int(os.environ.get("MQA_RANDOM_CASES", "1"))
SIZE = int(os.environ.get("MQA_RANDOM_SIZE", "1"))


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mqa_logits_amd  # noqa: F401


def _widen(bound, ref, out_dtype):
    if out_dtype != torch.bfloat16:
        return bound
    fin = np.isfinite(ref)
    return np.where(fin, bound + BF16_UNIT * (np.abs(np.where(fin, ref, 0.0)) + bound), bound)


def _draw(rng):
    fmt = ["fp8", "mxfp8", "mxfp4"][rng.integers(3)]
    h = int(rng.choice([8, 16, 32, 64]))
    d = int(rng.choice([64, 128]))
    out_dtype = torch.bfloat16 if rng.random() < 0.3 else torch.float32
    precision = "exact" if rng.random() < 0.25 else "default"
    return fmt, h, d, out_dtype, precision


def _ranges(rng, sq, skv):
    ks = rng.integers(-8, skv + 4, sq)
    ke = ks + rng.integers(-3, skv + 1, sq)
    kind = rng.integers(4)
    if kind == 1:                                   # causal-like
        ks[:] = 0
        ke = skv - sq + np.arange(sq) + 1
    elif kind == 2:                                 # full rows
        ks[:] = 0
        ke[:] = skv
    return ks.astype(np.int64), ke.astype(np.int64)


@pytest.mark.parametrize("seed", range(40 * SCALE))
def test_dense_and_compressed_random(seed):
    import mqa_logits_amd as mq
    rng = np.random.default_rng(7000 + seed)
    fmt, h, d, out_dtype, precision = _draw(rng)
    sq = int(rng.integers(1, 70))
    skv = int(rng.integers(1, 3000 * SIZE))
    ks, ke = _ranges(rng, sq, skv)
    clean = bool(rng.random() < 0.75)
    schedule = bool(rng.random() < 0.3)
    what = (f"seed{seed} {fmt} H{h} D{d} Sq{sq} Skv{skv} {str(out_dtype)[6:]} {precision} "
            f"clean={clean} sched={schedule}")
    log(f"[random] dense {what}")
    case = synth.dense_case(sq, skv, h, d, fmt, seed=8000 + seed, k_start=ks, k_end=ke)
    if fmt == "fp8" and rng.random() < 0.5:         # negative and zero token scales
        flip = rng.random(skv) < 0.3
        case.kv_scale[flip] *= -1.0
        case.kv_scale[rng.random(skv) < 0.05] = 0.0
    dd = dense_on_device(case)
    args = (dd["fmt"], dd["q"], dd["q_sf"], dd["kv"], dd["kv_sf"], dd["kv_scale"], dd["weights"],
            dd["k_start"], dd["k_end"])
    sched = mq.mqa_logits_metadata(dd["k_start"], dd["k_end"], skv, int(rng.integers(1, 300))) \
        if schedule else None
    # a row stride past the width, with guard columns that must survive
    pad = int(rng.integers(0, 9)) * (2 if out_dtype == torch.bfloat16 else 1)
    width = skv + pad + (skv & 1 if out_dtype == torch.bfloat16 else 0)
    buf = torch.full((sq, width), GUARD, dtype=out_dtype, device="cuda")
    out = buf[:, :skv]
    mq.mqa_logits(*args, clean_logits=clean, out=out, schedule=sched, logits_dtype=out_dtype,
                  precision=precision)
    packed, off = mq.mqa_logits_compressed(*args, schedule=sched, logits_dtype=out_dtype,
                                           precision=precision)
    torch.cuda.synchronize()
    host = buf.float().cpu().numpy().astype(np.float64)
    assert np.all(host[:, skv:] == GUARD), f"{what}: guard columns written"
    ref, bound = oracle.dense_logits(*case.args())
    b = _widen(bound, ref, out_dtype)
    got = host[:, :skv]
    if clean:
        assert_close(got, ref, b, what)
    else:
        inside = np.isfinite(ref)
        assert np.all(got[~inside] == GUARD), f"{what}: keep mode wrote outside the ranges"
        assert_close(np.where(inside, got, -np.inf), ref, b, what)
    cref, cbound, coff = oracle.compressed_logits(*case.args())
    assert np.array_equal(off.cpu().numpy(), coff), f"{what}: row offsets"
    assert_close(packed.float().cpu().numpy(), cref, _widen(cbound, cref, out_dtype),
                 f"{what} compressed")


@pytest.mark.parametrize("seed", range(20 * SCALE))
def test_paged_random(seed):
    import mqa_logits_amd as mq
    rng = np.random.default_rng(9000 + seed)
    fmt, h, d, out_dtype, precision = _draw(rng)
    batch = int(rng.integers(1, 6))
    next_n = int(rng.integers(1, 9 if SIZE == 1 else 17))
    bs = int(rng.choice([16, 32, 64]))
    max_ctx = int(rng.integers(1, 900 * SIZE))
    ctx = rng.integers(0, max_ctx + 80, batch)
    nb = -(-max_ctx // bs)
    num_blocks = batch * nb + int(rng.integers(0, 20))
    clean = bool(rng.random() < 0.75)
    splits = int(rng.integers(1, 400))
    what = (f"seed{seed} {fmt} H{h} D{d} batch{batch} next_n{next_n} bs{bs} max_ctx{max_ctx} "
            f"{str(out_dtype)[6:]} {precision} clean={clean} splits={splits}")
    log(f"[random] paged {what}")
    case = synth.paged_case(batch=batch, next_n=next_n, h=h, d=d, block_size=bs,
                            num_blocks=num_blocks, ctx_lo=0, ctx_hi=0, max_context_len=max_ctx,
                            fmt=fmt, seed=9500 + seed, context_lens=ctx)
    if fmt == "fp8" and rng.random() < 0.5:         # negative and zero token scales
        pool = case.kv_scale_pool
        sign = np.where(rng.random(pool.shape) < 0.3, -1.0, 1.0).astype(np.float32)
        case.kv_scale_pool = pool * sign
        case.kv_scale_pool[rng.random(pool.shape) < 0.05] = 0.0
    pd = paged_on_device(case)
    if rng.random() < 0.5:                          # a block table with a wider row stride
        wide = torch.full((batch, case.block_table.shape[1] + int(rng.integers(1, 7))), -1,
                          dtype=torch.int32, device="cuda")
        wide[:, :case.block_table.shape[1]] = pd["block_table"]
        pd["block_table"] = wide[:, :case.block_table.shape[1]]
    sched = mq.paged_mqa_logits_metadata(pd["context_lens"], next_n, bs, max_ctx, splits)
    rows = batch * next_n
    pad = int(rng.integers(0, 9)) * (2 if out_dtype == torch.bfloat16 else 1)
    width = max_ctx + pad + (max_ctx & 1 if out_dtype == torch.bfloat16 else 0)
    buf = torch.full((rows, width), GUARD, dtype=out_dtype, device="cuda")
    out = buf[:, :max_ctx]
    mq.paged_mqa_logits(fmt, pd["q"], pd["q_sf"], pd["kv_pool"], pd["kv_sf_pool"],
                        pd["kv_scale_pool"], pd["weights"], pd["context_lens"], pd["block_table"],
                        sched, next_n, max_ctx, clean_logits=clean, out=out,
                        logits_dtype=out_dtype, precision=precision)
    torch.cuda.synchronize()
    host = buf.float().cpu().numpy().astype(np.float64)
    assert np.all(host[:, max_ctx:] == GUARD), f"{what}: guard columns written"
    ref, bound = oracle.paged_logits(*case.args())
    b = _widen(bound, ref, out_dtype)
    got = host[:, :max_ctx]
    if clean:
        assert_close(got, ref, b, what)
    else:
        inside = np.isfinite(ref)
        assert np.all(got[~inside] == GUARD), f"{what}: keep mode wrote outside the ranges"
        assert_close(np.where(inside, got, -np.inf), ref, b, what)


@pytest.mark.parametrize("seed", range(20 * SCALE))
def test_topk_random(seed):
    # row lengths across every register-kernel capacity and the streaming
    # kernel, topk from 1 to past the row length, ties, fp32 and bf16 logits
    import mqa_logits_amd as mq
    rng = np.random.default_rng(9900 + seed)
    sq = int(rng.integers(1, 40))
    skv = int(rng.choice([int(rng.integers(1, 9000)), int(rng.integers(9000, 70000))]))
    topk = int(rng.choice([1, int(rng.integers(1, 5000)), 2048]))
    ties = bool(rng.random() < 0.6)
    ranges = bool(rng.random() < 0.7)
    bf16 = bool(rng.random() < 0.3)
    what = f"seed{seed} Sq{sq} Skv{skv} topk{topk} ties={ties} ranges={ranges} bf16={bf16}"
    log(f"[random] topk {what}")
    x, ks, ke = synth.topk_logits(sq, skv, 9950 + seed, ties=ties, ranges=ranges)
    t = dev(x)
    if bf16:
        bits = synth.encode_bf16(x)
        x = synth.decode_bf16(bits).reshape(x.shape)
        t = dev(bits.view(np.int16)).view(torch.bfloat16)
    if rng.random() < 0.5:                          # rows inside a wider buffer
        wide = torch.full((sq, skv + int(rng.integers(1, 9))), float("nan"), dtype=t.dtype,
                          device="cuda")
        wide[:, :skv] = t
        t = wide[:, :skv]
    got = mq.mqa_logits_topk(t, topk, dev(ks), dev(ke)).cpu().numpy()
    assert np.array_equal(got, oracle.topk_indices(x, topk, ks, ke)), what
