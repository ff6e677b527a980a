"""GPU checks of the dense work schedule (mqa_logits_metadata) and the
scheduled dense / compressed path.

The schedule must equal the oracle's split bit for bit.  The scheduled
output must be bitwise identical to the unscheduled one for every split count
(no work crosses a column, so the split cannot change a value), and match the
oracle element by element.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_helpers import assert_close, dense_on_device, dev, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mqa_logits_amd  # noqa: F401


def _ranges(kind, sq, skv, seed):
    rng = np.random.default_rng(seed)
    if kind == "causal":                       # prefill: row i sees [0, skv - sq + i + 1)
        return np.zeros(sq, np.int64), skv - sq + np.arange(sq) + 1
    if kind == "windows":                      # irregular windows, empty and reversed rows
        ks = rng.integers(-40, skv + 40, sq)
        ke = ks + rng.integers(-30, skv // 2, sq)
        ks[:3], ke[:3] = [7, 0, skv - 1], [7, skv, skv + 9]
        return ks, ke
    if kind == "cp":                           # one context-parallel shard's window
        lo = skv // 3
        return np.full(sq, lo), np.minimum(lo + np.arange(sq) * 3 + 1, skv)
    raise ValueError(kind)


@pytest.mark.parametrize("kind,sq,skv,splits", [
    ("windows", 37, 999, 7),
    ("causal", 2048, 32768, 1024),
    ("cp", 130, 5000, 1),
    ("windows", 32768, 300, 5000),
    ("causal", 1, 1, 64),
])
def test_dense_metadata_matches_oracle(kind, sq, skv, splits):
    import mqa_logits_amd as mq
    ks, ke = _ranges(kind, sq, skv, sq + splits)
    log(f"[schedule] metadata {kind} Sq={sq} Skv={skv} splits={splits}")
    got = mq.mqa_logits_metadata(dev(ks.astype(np.int32)), dev(ke.astype(np.int32)), skv, splits)
    ref = oracle.dense_schedule(ks, ke, skv, splits)
    assert np.array_equal(got.cpu().numpy(), ref)


def _both(case, splits, **kw):
    import mqa_logits_amd as mq
    d = dense_on_device(case)
    args = (d["fmt"], d["q"], d["q_sf"], d["kv"], d["kv_sf"], d["kv_scale"], d["weights"],
            d["k_start"], d["k_end"])
    sched = mq.mqa_logits_metadata(d["k_start"], d["k_end"], case.skv, splits)
    plain = mq.mqa_logits(*args, **kw)
    scheduled = mq.mqa_logits(*args, schedule=sched, **kw)
    torch.cuda.synchronize()
    return plain, scheduled


@pytest.mark.parametrize("fmt", ["fp8", "mxfp8", "mxfp4"])
@pytest.mark.parametrize("h,d", [(64, 128), (32, 64), (16, 64)])
def test_scheduled_equals_unscheduled_and_oracle(fmt, h, d):
    sq, skv = 70, 1500
    ks, ke = _ranges("windows", sq, skv, h + d)
    case = synth.dense_case(sq, skv, h, d, fmt, seed=300 + h, k_start=ks, k_end=ke)
    ref, bound = oracle.dense_logits(*case.args())
    for splits in (1, 9, 300):
        log(f"[schedule] {fmt} H={h} D={d} splits={splits}")
        plain, scheduled = _both(case, splits)
        assert torch.equal(plain.view(torch.int32), scheduled.view(torch.int32)), f"splits={splits}"
    assert_close(scheduled.cpu().numpy(), ref, bound, f"sched_{fmt}_h{h}_d{d}")


@pytest.mark.parametrize("kind", ["causal", "cp"])
def test_scheduled_causal_and_cp_window(kind):
    sq, skv = 512, 4096
    ks, ke = _ranges(kind, sq, skv, 5)
    case = synth.dense_case(sq, skv, 64, 128, "fp8", seed=21, k_start=ks, k_end=ke)
    log(f"[schedule] {kind} Sq={sq} Skv={skv}")
    plain, scheduled = _both(case, 1024)
    assert torch.equal(plain.view(torch.int32), scheduled.view(torch.int32))
    ref, bound = oracle.dense_logits(*case.args())
    assert_close(scheduled.cpu().numpy(), ref, bound, f"sched_{kind}")


def test_scheduled_keep_mode_and_bf16():
    sq, skv = 41, 777
    ks, ke = _ranges("windows", sq, skv, 9)
    case = synth.dense_case(sq, skv, 32, 128, "fp8", seed=22, k_start=ks, k_end=ke)
    log("[schedule] keep mode")
    import mqa_logits_amd as mq
    d = dense_on_device(case)
    args = (d["fmt"], d["q"], d["q_sf"], d["kv"], d["kv_sf"], d["kv_scale"], d["weights"],
            d["k_start"], d["k_end"])
    sched = mq.mqa_logits_metadata(d["k_start"], d["k_end"], skv, 13)
    a = torch.full((sq, skv), 5.5, dtype=torch.float32, device="cuda")
    b = a.clone()
    mq.mqa_logits(*args, clean_logits=False, out=a)
    mq.mqa_logits(*args, clean_logits=False, out=b, schedule=sched)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    log("[schedule] bf16 logits")
    p16, s16 = _both(case, 13, logits_dtype=torch.bfloat16)
    assert torch.equal(p16.view(torch.int16), s16.view(torch.int16))


@pytest.mark.parametrize("fmt,h,d", [("mxfp4", 64, 128), ("fp8", 32, 64), ("mxfp8", 32, 64)])
def test_scheduled_compressed_equals_unscheduled(fmt, h, d):
    import mqa_logits_amd as mq
    sq, skv = 66, 2000
    ks, ke = _ranges("windows", sq, skv, 3)
    case = synth.dense_case(sq, skv, h, d, fmt, seed=23, k_start=ks, k_end=ke)
    d = dense_on_device(case)
    args = (d["fmt"], d["q"], d["q_sf"], d["kv"], d["kv_sf"], d["kv_scale"], d["weights"],
            d["k_start"], d["k_end"])
    sched = mq.mqa_logits_metadata(d["k_start"], d["k_end"], skv, 50)
    log(f"[schedule] compressed {fmt} H={h} D={d}")
    plain, off = mq.mqa_logits_compressed(*args)
    scheduled, _ = mq.mqa_logits_compressed(*args, row_offsets=off, schedule=sched)
    torch.cuda.synchronize()
    assert torch.equal(plain.view(torch.int32), scheduled.view(torch.int32))
    ref, bound, _ = oracle.compressed_logits(*case.args())
    assert_close(scheduled.cpu().numpy(), ref, bound, f"sched_compressed_{fmt}_h{h}_d{d}")
