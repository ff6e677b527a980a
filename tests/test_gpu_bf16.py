"""GPU parity with bf16 weights and/or bf16 logits (dense, compressed, paged).

bf16 weights are an input format: the oracle takes the exact values of the
bf16 bits the device reads.  bf16 logits are the fp32 results rounded to
nearest even, so against the oracle each in-range entry may differ by the fp32
bound plus the rounding, |bf16 - fp32| <= 2^-8 |fp32| <= 2^-8 (|ref| + bound);
-inf must stay exactly -inf.  Independently of the oracle, the bf16 logits
must be bit for bit torch's bf16 rounding of the library's own fp32 logits on
the same inputs (the arithmetic before the store is the same).
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_helpers import assert_close, dense_on_device, dev, log, paged_on_device

pytestmark = pytest.mark.gpu

BF16_UNIT = 2.0 ** -8          # relative rounding bound of bf16 (8 significant bits)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mqa_logits_amd  # noqa: F401


def _bf16_weights(case):
    """Round the case's weights to bf16: the oracle sees the bf16 values, the
    device gets the bf16 tensor."""
    bits = synth.encode_bf16(case.weights)
    case.weights = synth.decode_bf16(bits).reshape(case.weights.shape)
    return dev(bits.view(np.int16)).view(torch.bfloat16)


def _compare(out, ref, bound, what, clean=True):
    got = out.float().cpu().numpy().astype(np.float64)
    if out.dtype == torch.bfloat16:
        fin = np.isfinite(ref)
        bound = np.where(fin, bound + BF16_UNIT * (np.abs(np.where(fin, ref, 0.0)) + bound), bound)
    return assert_close(got, ref, bound, what, clean=clean)


def _dense(case, w_bf16, out_bf16, clean=True, out=None):
    import mqa_logits_amd as mq
    d = dense_on_device(case)
    if w_bf16:
        d["weights"] = _bf16_weights(case)
    dt = torch.bfloat16 if out_bf16 else torch.float32
    res = mq.mqa_logits(d["fmt"], d["q"], d["q_sf"], d["kv"], d["kv_sf"], d["kv_scale"],
                        d["weights"], d["k_start"], d["k_end"], clean_logits=clean, out=out,
                        logits_dtype=dt)
    torch.cuda.synchronize()
    return res, d


TYPES = [(True, False), (False, True), (True, True)]


@pytest.mark.parametrize("w_bf16,out_bf16", TYPES)
@pytest.mark.parametrize("fmt", ["fp8", "mxfp8", "mxfp4"])
@pytest.mark.parametrize("h,d", [(64, 128), (32, 64), (16, 64)])
def test_dense_bf16_matrix(fmt, h, d, w_bf16, out_bf16):
    sq, skv = 37, 999                     # odd Skv: ragged last group, padded bf16 stride
    ks = np.arange(sq) * 7 - 20
    ke = skv - 60 + np.arange(sq) * 2
    ke[3] = ks[3]                          # an empty row
    case = synth.dense_case(sq, skv, h, d, fmt, seed=200 + h + d, k_start=ks, k_end=ke)
    what = f"bf16_{fmt}_h{h}_d{d}_w{int(w_bf16)}_o{int(out_bf16)}"
    log(f"[bf16] {what}")
    out, _ = _dense(case, w_bf16, out_bf16)
    assert out.dtype == (torch.bfloat16 if out_bf16 else torch.float32)
    ref, bound = oracle.dense_logits(*case.args())
    _compare(out, ref, bound, what)


@pytest.mark.parametrize("sq,skv", [(129, 4100), (5, 17), (1, 1), (64, 16)])
def test_dense_bf16_logits_are_rounded_fp32_logits(sq, skv):
    import mqa_logits_amd as mq
    rng = np.random.default_rng(sq + skv)
    ks = rng.integers(-5, skv, sq)
    ke = ks + rng.integers(-3, skv + 5, sq)
    case = synth.dense_case(sq, skv, 64, 128, "fp8", seed=sq * skv, k_start=ks, k_end=ke)
    d = dense_on_device(case)
    log(f"[bf16] rounding identity {sq}x{skv}")
    args = (d["fmt"], d["q"], d["q_sf"], d["kv"], d["kv_sf"], d["kv_scale"], d["weights"],
            d["k_start"], d["k_end"])
    f32 = mq.mqa_logits(*args)
    b16 = mq.mqa_logits(*args, logits_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    want = f32.to(torch.bfloat16)
    assert torch.equal(b16.view(torch.int16), want.view(torch.int16))
    ref, bound = oracle.dense_logits(*case.args())
    _compare(b16, ref, bound, f"bf16_round_{sq}x{skv}")


def test_dense_bf16_keep_mode_and_guard_columns():
    sq, skv, stride = 40, 501, 520
    ks = np.arange(sq) * 5
    ke = ks + 200
    case = synth.dense_case(sq, skv, 64, 128, "mxfp8", seed=41, k_start=ks, k_end=ke)
    sentinel = 7.0                          # exact in bf16
    buf = torch.full((sq + 1, stride), sentinel, dtype=torch.bfloat16, device="cuda")
    log("[bf16] keep mode")
    _dense(case, True, True, clean=False, out=buf[:sq, :skv])
    b = buf.float().cpu().numpy()
    assert np.all(b[:sq, skv:] == sentinel) and np.all(b[sq] == sentinel)
    ref, bound = oracle.dense_logits(*case.args())
    inside = np.isfinite(ref)
    got = b[:sq, :skv]
    assert np.all(got[~inside] == sentinel)
    masked = torch.from_numpy(np.where(inside, got, -np.inf)).to(torch.bfloat16)
    _compare(masked, ref, bound, "bf16_keep")


@pytest.mark.parametrize("fmt", ["fp8", "mxfp8", "mxfp4"])
def test_compressed_bf16(fmt):
    import mqa_logits_amd as mq
    sq, skv = 70, 1501
    rng = np.random.default_rng(13)
    ks = rng.integers(-10, skv, sq)
    ke = ks + rng.integers(-5, 700, sq)
    case = synth.dense_case(sq, skv, 32, 64, fmt, seed=31, k_start=ks, k_end=ke)
    d = dense_on_device(case)
    w = _bf16_weights(case)
    off = mq.mqa_logits_compressed_offsets(d["k_start"], d["k_end"], skv)
    total = int(off[-1].item())
    buf = torch.full((total + 33,), -3.0, dtype=torch.bfloat16, device="cuda")
    log(f"[bf16] compressed {fmt}")
    mq.mqa_logits_compressed(d["fmt"], d["q"], d["q_sf"], d["kv"], d["kv_sf"], d["kv_scale"], w,
                             d["k_start"], d["k_end"], row_offsets=off, out=buf[1:total + 1])
    torch.cuda.synchronize()
    b = buf.float().cpu().numpy()
    assert b[0] == -3.0 and np.all(b[total + 1:] == -3.0)      # odd start, guard band
    ref, bound, ref_off = oracle.compressed_logits(*case.args())
    assert np.array_equal(off.cpu().numpy(), ref_off)
    _compare(buf[1:total + 1], ref, bound, f"bf16_compressed_{fmt}")


@pytest.mark.parametrize("fmt,next_n,bs", [("fp8", 3, 32), ("mxfp4", 2, 64), ("mxfp8", 6, 16)])
def test_paged_bf16(fmt, next_n, bs):
    import mqa_logits_amd as mq
    case = synth.paged_case(batch=5, next_n=next_n, h=64, d=128, block_size=bs, num_blocks=600,
                            ctx_lo=1, ctx_hi=1500, max_context_len=1603, fmt=fmt, seed=70 + bs,
                            context_lens=[2, 700, 1603, 33, 1025])
    d = paged_on_device(case)
    w = _bf16_weights(case)
    sched = mq.paged_mqa_logits_metadata(d["context_lens"], next_n, bs, case.max_context_len, 29)
    log(f"[bf16] paged {fmt} next_n={next_n} bs={bs}")
    out = mq.paged_mqa_logits(fmt, d["q"], d["q_sf"], d["kv_pool"], d["kv_sf_pool"],
                              d["kv_scale_pool"], w, d["context_lens"], d["block_table"], sched,
                              next_n, case.max_context_len, logits_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert out.dtype == torch.bfloat16 and out.stride(0) % 2 == 0
    ref, bound = oracle.paged_logits(*case.args())
    _compare(out, ref, bound, f"bf16_paged_{fmt}")
