"""Throughput of the weighted MQA-logits hot path on one MI355X.

Default workload: dense clean logits, Sq=2048 query rows, Skv=32768 keys,
H=64 heads, D=128, fp8 e4m3 Q/KV with fp32 per-token scales and weights, row i
covering keys [0, Skv - Sq + i) -- the indexer prefill shape.  One step = one
full call of the path on inputs already resident in HBM.  Metric: effective
TFLOP/s = 2 * H * D * (in-range entries) / time; masked and -inf entries are
not counted.

Order of work (all on cuda:0, one JSON line on stdout):
  1. inputs, one call and the full -inf mask check;
  2. cold window: the next 20 calls, timed together (reported, not the value);
  3. graph replay: 5 calls with distinct outputs captured in one HIP graph,
     5 replays, then 40 samples of an untimed replay followed by an
     event-timed one; median, p10 and p90 per call (reported);
  4. W warmup steps, then exactly K steps between a barrier-free pair of HIP
     events, with host wall time around them: `value` is the effective
     TFLOP/s over the wall time, `roofline.achieved` over the event time;
  5. the MFMA microbenchmark (rate and the clock its waves ran at), and the
     CPU oracle on a bounded sample.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c1]
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MQA-logits effective TFLOP/s + % fp8 MFMA peak (H64 D128, 2K×32K)"

# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s)
PEAK_TFLOPS = {"fp8": 5000.0, "mxfp8": 5000.0, "mxfp4": 10100.0}
PEAK_HBM_GBS = 8000.0

WORKLOADS = {"c0": 0, "c1": 1, "c2": 2, "c3": 3, "c4-mxfp8": 4, "c4-mxfp4": 4,
             "c1-mxfp8": 1, "c1-mxfp4": 1, "c3-mxfp8": 3, "c3-mxfp4": 3}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_digest(names):
    """sha256 over the named files of mqa_logits_amd/csrc, so traffic counted
    for older kernels is not reused."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mqa_logits_amd", "csrc")
    for name in sorted(names):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    counter summary (profiles/<kernel>_<workload>_traffic.txt), if it was taken
    on the current kernel sources; None otherwise."""
    import glob
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", f"*_{workload}_traffic.txt")))
    if not paths:
        return None
    path = paths[0]
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    names = fields.get("sources", "").split()
    try:
        if not names or fields.get("source_sha256") != kernel_source_digest(names):
            return None
    except OSError:
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def mfma_microbench():
    """Dense fp8 MFMA rate and shader clock from libmqa_peak.so (one wave per
    SIMD, chains of the same MFMA the kernels use); None if unavailable."""
    import ctypes
    import mqa_logits_amd as mq
    path = os.path.join(os.path.dirname(mq.LIB_PATH), "libmqa_peak.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    fn = lib.mqa_measure_mfma_peak
    fn.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_double),
                   ctypes.POINTER(ctypes.c_double)]
    fn.restype = ctypes.c_int
    t, c = ctypes.c_double(), ctypes.c_double()
    if fn(mq.mqa_num_cus(0) * 4, 4000, ctypes.byref(t), ctypes.byref(c)) != 0:
        return None
    return {"tflops": t.value, "sclk_mhz": c.value}


def clamped_ranges(k_start, k_end, skv):
    """Row ranges as the metric counts them: [clamp(s,0,Skv), clamp(e,s,Skv))."""
    s = np.clip(np.asarray(k_start, np.int64), 0, skv)
    return s, np.clip(np.asarray(k_end, np.int64), s, skv)


def valid_entries_dense(case):
    s, e = clamped_ranges(case.k_start, case.k_end, case.skv)
    return int((e - s).sum())


def check_mask(out, case, rows_per_chunk=128):
    """-inf exactly outside each row's range, finite inside (checked before timing)."""
    import torch
    s, e = clamped_ranges(case.k_start, case.k_end, case.skv)
    S, E = torch.from_numpy(s).cuda(), torch.from_numpy(e).cuda()
    cols = torch.arange(case.skv, device="cuda")
    for r0 in range(0, case.sq, rows_per_chunk):
        r1 = min(r0 + rows_per_chunk, case.sq)
        valid = (cols[None, :] >= S[r0:r1, None]) & (cols[None, :] < E[r0:r1, None])
        chunk = out[r0:r1]
        if not (torch.equal(torch.isneginf(chunk), ~valid) and bool(torch.isfinite(chunk[valid]).all())):
            raise SystemExit(f"mask check failed in rows [{r0}, {r1})")


def build_step(name, schedule=False, logits_dtype="fp32", zero=False, precision="default"):
    """Returns (step_fn, info) with inputs resident on cuda:0.

    info["call"](o) makes one full call of the path writing into output buffer
    o; info["outs"] are distinct output buffers (5, or 2 for the 2 GiB
    outputs); step() calls into them in turn.  schedule: dense / compressed
    calls follow a work schedule made by mqa_logits_metadata once, outside the
    steps (its own time is reported as metadata_ms).  logits_dtype: fp32 or
    bf16 logits."""
    import torch
    import mqa_logits_amd as mq
    import synth

    out_dtype = {"fp32": torch.float32, "bf16": torch.bfloat16}[logits_dtype]
    out_size = 4 if logits_dtype == "fp32" else 2

    idx = WORKLOADS[name]
    fmt = name.split("-")[1] if "-" in name else None
    case = synth.workload_case(idx, fmt, zero=zero)
    dev = lambda x: None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()
    info = dict(workload=case.name + ("_zero" if zero else ""), case=case)
    n_out = 2 if idx == 4 else 5

    def rotating(call, outs):
        state = {"i": 0}

        def step():
            call(outs[state["i"] % len(outs)])
            state["i"] += 1
        return step

    def dense_schedule(ks, ke):
        if not schedule:
            return None, {}
        splits = mq.paged_mqa_logits_default_splits(0)
        sched = mq.mqa_logits_metadata(ks, ke, case.skv, splits)

        def metadata_ms(n=50):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(n):
                mq.mqa_logits_metadata(ks, ke, case.skv, splits, out=sched)
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b) / n
        return sched, dict(extra=lambda: {"metadata_ms": metadata_ms()})

    if idx in (0, 1, 4):
        d = [dev(x) for x in case.args()[1:]]
        q, q_sf, kv, kv_sf, kvs, w, ks, ke = d
        sched, extra = dense_schedule(ks, ke)
        outs = [mq._logits_rows(case.sq, case.skv, out_dtype, "cuda") for _ in range(n_out)]

        def call(o):
            mq.mqa_logits(case.fmt, q, q_sf, kv, kv_sf, kvs, w, ks, ke, out=o, schedule=sched,
                          precision=precision)
        nvalid = valid_entries_dense(case)
        info["topk"] = lambda k: time_topk(lambda: mq.mqa_logits_topk(outs[0], k, ks, ke),
                                           nvalid * out_size + case.sq * k * 4)
        info.update(flops=2.0 * case.h * case.d * nvalid, fmt=case.fmt, bound="mfma",
                    out_bytes=float(out_size) * case.sq * case.skv, call=call, outs=outs,
                    cfg=dict(sq=case.sq, skv=case.skv, heads=case.h, head_dim=case.d,
                             format=case.fmt, layout="dense", clean_logits=True,
                             logits=logits_dtype, schedule=bool(schedule)), **extra)
        # mask check before timing (the pages' reproducer checks the mask too)
        call(outs[0])
        torch.cuda.synchronize()
        check_mask(outs[0], case)
        return rotating(call, outs), info

    if idx == 2:
        d = [dev(x) for x in case.args()[1:]]
        q, q_sf, kv, kv_sf, kvs, w, ks, ke = d
        off = mq.mqa_logits_compressed_offsets(ks, ke, case.skv)
        total = int(off[-1].item())
        sched, extra = dense_schedule(ks, ke)
        outs = [torch.empty(total, dtype=out_dtype, device="cuda") for _ in range(n_out)]

        def call(o):
            mq.mqa_logits_compressed_offsets(ks, ke, case.skv, out=off)
            mq.mqa_logits_compressed(case.fmt, q, q_sf, kv, kv_sf, kvs, w, ks, ke,
                                     row_offsets=off, out=o, schedule=sched,
                                     precision=precision)
        nvalid = valid_entries_dense(case)
        info.update(flops=2.0 * case.h * case.d * nvalid, fmt=case.fmt, bound="mfma",
                    out_bytes=float(out_size) * total, call=call, outs=outs,
                    cfg=dict(sq=case.sq, skv=case.skv, heads=case.h, head_dim=case.d,
                             format=case.fmt, layout="compressed", logits=logits_dtype,
                             schedule=bool(schedule)), **extra)
        return rotating(call, outs), info

    # paged decode
    pd = dict(q=dev(case.q), q_sf=dev(case.q_sf), kv=dev(case.kv_pool),
              kv_sf=dev(case.kv_sf_pool), kvs=dev(case.kv_scale_pool), w=dev(case.weights),
              ctx=dev(case.context_lens), bt=dev(case.block_table))
    splits = mq.paged_mqa_logits_default_splits(0)
    sched = mq.paged_mqa_logits_metadata(pd["ctx"], case.next_n, case.block_size,
                                         case.max_context_len, splits)
    rows = case.batch * case.next_n
    outs = [mq._logits_rows(rows, case.max_context_len, out_dtype, "cuda") for _ in range(n_out)]

    # The schedule is made once per decoding step and shared by every layer's
    # kernel: it is timed on its own, outside the steps.
    def call(o):
        mq.paged_mqa_logits(case.fmt, pd["q"], pd["q_sf"], pd["kv"], pd["kv_sf"], pd["kvs"],
                            pd["w"], pd["ctx"], pd["bt"], sched, case.next_n,
                            case.max_context_len, out=o, precision=precision)

    def metadata_ms(n=50):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            mq.paged_mqa_logits_metadata(pd["ctx"], case.next_n, case.block_size,
                                         case.max_context_len, splits, out=sched)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n
    ctx = np.asarray(case.context_lens, np.int64)
    length = np.minimum(ctx, case.max_context_len)
    t = np.arange(case.next_n)
    nvalid = int(np.clip(ctx[:, None] - case.next_n + t[None, :] + 1, 0, length[:, None]).sum())
    n_units = int(((length + case.block_size - 1) // case.block_size).sum())
    row_bytes = case.d * (1 if case.fmt != "mxfp4" else 0.5)
    kv_bytes = n_units * case.block_size * (row_bytes + 4)
    out_bytes = rows * case.max_context_len * out_size
    # top-k over whole rows: the -inf past each row's range is not a candidate
    info["topk"] = lambda k: time_topk(lambda: mq.mqa_logits_topk(outs[0], k),
                                       out_bytes + rows * k * 4)
    info.update(flops=2.0 * case.h * case.d * nvalid, fmt=case.fmt, bound="hbm",
                out_bytes=out_bytes, extra=lambda: {"metadata_ms": metadata_ms()},
                bytes=kv_bytes + out_bytes + case.q.nbytes + case.weights.nbytes,
                call=call, outs=outs,
                cfg=dict(batch=case.batch, next_n=case.next_n, heads=case.h, head_dim=case.d,
                         block_size=case.block_size, max_context_len=case.max_context_len,
                         format=case.fmt, layout="paged", splits=splits, logits=logits_dtype))
    return rotating(call, outs), info


def graph_protocol(call, outs, samples=40):
    """The pages' timing method: 3 warm-up calls; one HIP graph holding one
    call per distinct output buffer; 5 replays; then `samples` times an
    untimed replay followed by an event-timed one.  Returns per-call median,
    p10 and p90 in ms."""
    import statistics
    import torch
    for _ in range(3):
        call(outs[0])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for o in outs:
            call(o)
    for _ in range(5):
        g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for _ in range(samples):
        g.replay()
        a.record()
        g.replay()
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b) / len(outs))
    srt = sorted(times)
    return {"calls_per_graph": len(outs), "samples": samples,
            "median_ms": statistics.median(times), "p10_ms": srt[int(0.1 * (samples - 1))],
            "p90_ms": srt[int(0.9 * (samples - 1))]}


def time_topk(fn, nbytes, n=50):
    """Average time of the top-k selection over a step's logits (HIP events
    around n back-to-back calls) and the rate of its algorithmic bytes
    (logits read once + indices written)."""
    import torch
    for _ in range(5):
        fn()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(n):
        fn()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / n
    return {"ms": ms, "algorithmic_bytes": nbytes, "gbs": nbytes / (ms * 1e-3) / 1e9}


def cpu_baseline(info, seconds):
    """The oracle, as it stands, on leading rows of the same workload for about
    `seconds` of wall time with every BLAS thread the process has; plus the
    extrapolated time of the whole workload and, for scale, the whole tiny
    workload (256 x 1024, H 16, D 64) on one thread."""
    import oracle                          # the oracle is used by this leg only
    import synth
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threadpool_limits = None
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    case = info["case"]
    if not hasattr(case, "sq"):
        return None
    s, e = clamped_ranges(case.k_start, case.k_end, case.skv)
    t0 = time.perf_counter()
    done, flops, block = 0, 0.0, 8
    while done < case.sq and time.perf_counter() - t0 < seconds:
        rows = np.arange(done, min(done + block, case.sq))
        oracle.dense_logits(*case.args(), rows=rows, row_block=block)
        flops += 2.0 * case.h * case.d * float((e[rows] - s[rows]).sum())
        done = rows[-1] + 1
    dt = time.perf_counter() - t0
    out = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "sample": f"rows 0..{done - 1} of the same workload (float64 numpy oracle), "
                     f"{dt:.1f} s wall",
           "rows_per_s": done / dt,
           "extrapolated_full_workload_s": dt * info["flops"] / flops if flops else None}
    if threadpool_limits is not None:
        tiny = synth.workload_case(0)
        with threadpool_limits(limits=1):
            t1 = time.perf_counter()
            oracle.dense_logits(*tiny.args())
            out["tiny_workload_one_thread_s"] = time.perf_counter() - t1
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c1", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-replay protocol")
    ap.add_argument("--schedule", action="store_true",
                    help="dense/compressed calls follow an mqa_logits_metadata work schedule")
    ap.add_argument("--logits-dtype", default="fp32", choices=["fp32", "bf16"])
    ap.add_argument("--precision", default="default", choices=["default", "exact"])
    ap.add_argument("--zero", action="store_true",
                    help="all-zero Q, KV and weights with unit scales (the pages' timing "
                         "workload; dense workloads only)")
    ap.add_argument("--topk", type=int, default=0, metavar="K",
                    help="also time mqa_logits_topk(K) over a step's logits (reported apart)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB per step (the reference "
                         "point that scales HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards without communication; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": 4 * n, "bytes_written": 4 * n,
                          "launches": args.warmup + args.steps}), flush=True)
        return
    step, info = build_step(args.workload, args.schedule, args.logits_dtype, args.zero,
                            args.precision)
    if args.zero:
        info["cfg"]["inputs"] = "all_zero"
    if args.precision != "default":
        info["cfg"]["precision"] = args.precision
    flops = info["flops"]
    stream = torch.cuda.current_stream()

    def timed(n):
        """n back-to-back steps between two HIP events on the launch stream;
        (host wall s, event ms per step)."""
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        a.record(stream)
        for _ in range(n):
            step()
        b.record(stream)
        b.synchronize()
        wall = time.perf_counter() - t0
        return wall, a.elapsed_time(b) / n

    # cold window: the first calls after setup (the shader clock dips for
    # tens of milliseconds once sustained load starts)
    _, cold_ms = timed(20)
    graph = None if args.no_graph else graph_protocol(info["call"], info["outs"])

    for _ in range(args.warmup):
        step()
    # timed region (an event per step would put a cache-flushing marker between
    # the launches and time that too)
    wall, per_launch_ms = timed(args.steps)

    value = flops * args.steps / wall / 1e12
    # the committed counter summaries cover the default call
    default_call = (not args.schedule and args.logits_dtype == "fp32"
                    and args.precision == "default" and not args.zero)
    traffic = measured_traffic(args.workload) if default_call else None
    if info["bound"] == "mfma":
        achieved = flops / (per_launch_ms * 1e-3) / 1e12
        peak = PEAK_TFLOPS[info["fmt"]]
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak, "traffic": traffic}
    else:
        achieved = info["bytes"] / (per_launch_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": traffic}

    peak_probe = mfma_microbench()
    cpu = None if args.no_cpu_baseline else cpu_baseline(info, args.cpu_seconds)
    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"fp8": "fp8_e4m3", "mxfp8": "mxfp8_e4m3", "mxfp4": "mxfp4_e2m1"}[info["fmt"]],
        "data": "synthetic",
        "config": {"workload": info["workload"], **info["cfg"]},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernel_ms": per_launch_ms,
        "cold_window": {"calls": 20, "ms_per_call": cold_ms,
                        "frac": (flops / (cold_ms * 1e-3) / 1e12 / PEAK_TFLOPS[info["fmt"]]
                                 if info["bound"] == "mfma" else None)},
        "graph_replay": graph,
        "mfma_microbench": peak_probe,
        "hbm_write_gbs": info["out_bytes"] / (per_launch_ms * 1e-3) / 1e9,
    }
    if "extra" in info:
        line.update(info["extra"]())
    if args.topk and "topk" in info:
        line["topk"] = {"k": args.topk, **info["topk"](args.topk)}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
