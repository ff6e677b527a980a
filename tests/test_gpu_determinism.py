"""Bitwise repeatability and HIP-graph capture of the HIP path.

  * 20 calls with the same inputs give bit-identical outputs ("[PR #435]
    Improve SM100 MX MQA logits clean-output performance", Validation: the
    20-repeat bitwise checks), for the dense MX formats, the compressed
    layout, bf16 logits, the exact-products precision and the paged path;
  * a call captured into a torch.cuda.CUDAGraph on a side stream replays bit
    for bit like the eager call, several replays with eager work and
    synchronizations between them (the library allocates nothing and never
    waits, so every entry point can be captured).
"""

import numpy as np
import pytest
import torch

import synth
from tests.gpu_helpers import dense_on_device, log, paged_on_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mqa_logits_amd  # noqa: F401


def _bits(t):
    return t.contiguous().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).clone()


def _repeat(fn, n=20):
    first = _bits(fn())
    for _ in range(n - 1):
        assert torch.equal(_bits(fn()), first)


def _dense_fn(case, **kw):
    import mqa_logits_amd as mq
    d = dense_on_device(case)
    return lambda: mq.mqa_logits(d["fmt"], d["q"], d["q_sf"], d["kv"], d["kv_sf"], d["kv_scale"],
                                 d["weights"], d["k_start"], d["k_end"], **kw)


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_dense_mx_20_repeats(fmt):
    case = synth.dense_case(64, 5000, 64, 128, fmt, seed=21, k_end=4000 + np.arange(64) * 10)
    log(f"[determinism] dense {fmt}")
    _repeat(_dense_fn(case))


@pytest.mark.parametrize("h", [32, 64])
def test_dense_exact_products_20_repeats(h):
    case = synth.dense_case(48, 3000, h, 128, "fp8", seed=22, k_end=2500 + np.arange(48) * 7)
    log(f"[determinism] dense exact H={h}")
    _repeat(_dense_fn(case, precision="exact"))


def test_dense_bf16_logits_and_weights_20_repeats():
    import mqa_logits_amd as mq
    case = synth.dense_case(40, 2000, 64, 128, "fp8", seed=23, k_start=np.arange(40) * 9)
    d = dense_on_device(case)
    w = d["weights"].to(torch.bfloat16)
    log("[determinism] dense bf16")
    _repeat(lambda: mq.mqa_logits("fp8", d["q"], None, d["kv"], None, d["kv_scale"], w,
                                  d["k_start"], d["k_end"], logits_dtype=torch.bfloat16))


def test_compressed_20_repeats():
    import mqa_logits_amd as mq
    case = synth.dense_case(300, 1200, 32, 64, "fp8", seed=24, k_start=np.arange(300) * 4,
                            k_end=np.full(300, 1200))
    d = dense_on_device(case)
    off = mq.mqa_logits_compressed_offsets(d["k_start"], d["k_end"], case.skv)
    log("[determinism] compressed")
    _repeat(lambda: mq.mqa_logits_compressed("fp8", d["q"], None, d["kv"], None, d["kv_scale"],
                                             d["weights"], d["k_start"], d["k_end"],
                                             row_offsets=off)[0])


@pytest.mark.parametrize("fmt", ["fp8", "mxfp8"])
def test_paged_20_repeats(fmt):
    import mqa_logits_amd as mq
    case = synth.paged_case(16, 4, 64, 128, 64, 600, 300, 4000, 4096, fmt, seed=25)
    d = paged_on_device(case)
    sched = mq.paged_mqa_logits_metadata(d["context_lens"], 4, 64, 4096, 256)
    log(f"[determinism] paged {fmt}")
    _repeat(lambda: mq.paged_mqa_logits(fmt, d["q"], d["q_sf"], d["kv_pool"], d["kv_sf_pool"],
                                        d["kv_scale_pool"], d["weights"], d["context_lens"],
                                        d["block_table"], sched, 4, 4096))


def _graph_replays_equal_eager(fn, replays=3):
    """Capture fn (which writes into fixed output buffers and returns them) on a
    side stream, replay it several times with eager work and synchronizations
    between, and compare every replay with the eager result bit for bit."""
    eager = [_bits(t) for t in fn()]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                                      # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        outs = fn()
    torch.cuda.synchronize()
    for k in range(replays):
        for t in outs:
            t.fill_(float("nan") if t.is_floating_point() else -7)   # poison between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, eager):
            assert torch.equal(_bits(a), b), f"replay {k} differs"
        _ = torch.ones(1000, device="cuda").sum()          # unrelated eager work
        torch.cuda.synchronize()


def test_graph_capture_dense_h64():
    import mqa_logits_amd as mq
    case = synth.dense_case(96, 4100, 64, 128, "fp8", seed=26, k_end=4000 + np.arange(96))
    d = dense_on_device(case)
    out = torch.empty(96, 4100, device="cuda")
    log("[graph] dense H=64 capture and replay")
    _graph_replays_equal_eager(lambda: [mq.mqa_logits(
        "fp8", d["q"], None, d["kv"], None, d["kv_scale"], d["weights"], d["k_start"],
        d["k_end"], out=out)])


def test_graph_capture_scheduled_compressed_and_topk():
    import mqa_logits_amd as mq
    case = synth.dense_case(120, 3000, 64, 128, "mxfp8", seed=27, k_start=np.arange(120) * 5,
                            k_end=np.full(120, 3000))
    d = dense_on_device(case)
    sched = mq.mqa_logits_metadata(d["k_start"], d["k_end"], case.skv, 128)
    off = mq.mqa_logits_compressed_offsets(d["k_start"], d["k_end"], case.skv)
    total = int(off[-1].item())
    packed = torch.empty(total, device="cuda")
    dense_out = torch.empty(120, 3000, device="cuda")
    idx = torch.empty(120, 64, dtype=torch.int32, device="cuda")

    def fn():
        mq.mqa_logits_compressed_offsets(d["k_start"], d["k_end"], case.skv, out=off)
        mq.mqa_logits_compressed("mxfp8", d["q"], d["q_sf"], d["kv"], d["kv_sf"], None,
                                 d["weights"], d["k_start"], d["k_end"], row_offsets=off,
                                 out=packed, schedule=sched)
        mq.mqa_logits("mxfp8", d["q"], d["q_sf"], d["kv"], d["kv_sf"], None, d["weights"],
                      d["k_start"], d["k_end"], out=dense_out, schedule=sched)
        mq.mqa_logits_topk(dense_out, 64, d["k_start"], d["k_end"], out=idx)
        return [packed, dense_out, idx]
    log("[graph] scheduled compressed + dense + top-k capture and replay")
    _graph_replays_equal_eager(fn)


def test_graph_capture_paged():
    import mqa_logits_amd as mq
    case = synth.paged_case(8, 4, 64, 128, 64, 400, 200, 3000, 3072, "fp8", seed=28)
    d = paged_on_device(case)
    sched = torch.empty(257, 2, dtype=torch.int32, device="cuda")
    out = torch.empty(32, 3072, device="cuda")

    def fn():
        mq.paged_mqa_logits_metadata(d["context_lens"], 4, 64, 3072, 256, out=sched)
        mq.paged_mqa_logits("fp8", d["q"], None, d["kv_pool"], None, d["kv_scale_pool"],
                            d["weights"], d["context_lens"], d["block_table"], sched, 4, 3072,
                            out=out)
        return [sched, out]
    log("[graph] paged metadata + logits capture and replay")
    _graph_replays_equal_eager(fn)
