"""Helpers for the GPU parity tests: move seeded inputs to the device, run the
HIP path through the binding, and compare with the oracle.

Comparison rules (test infrastructure):
  * the -inf mask must match the oracle's exactly (clean logits);
  * every in-range GPU value must be finite and within the oracle's bound
    |gpu - ref| <= 1e-4 * sum_h |w * kv_scale * <q, kv>| + 1e-6;
  * indices (compressed offsets, paged schedule) must match bit for bit.
"""

import sys

import numpy as np
import torch

import oracle

DEVICE = "cuda"


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x):
    if x is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEVICE)


def dense_on_device(case):
    return dict(fmt=case.fmt, q=dev(case.q), q_sf=dev(case.q_sf), kv=dev(case.kv),
                kv_sf=dev(case.kv_sf), kv_scale=dev(case.kv_scale), weights=dev(case.weights),
                k_start=dev(case.k_start), k_end=dev(case.k_end))


def paged_on_device(case):
    return dict(fmt=case.fmt, q=dev(case.q), q_sf=dev(case.q_sf), kv_pool=dev(case.kv_pool),
                kv_sf_pool=dev(case.kv_sf_pool), kv_scale_pool=dev(case.kv_scale_pool),
                weights=dev(case.weights), context_lens=dev(case.context_lens),
                block_table=dev(case.block_table))


def assert_close(gpu, ref, bound, what, clean=True):
    """gpu: float32 array; ref/bound: oracle float64 arrays of the same shape."""
    gpu = np.asarray(gpu, dtype=np.float64)
    inf_ref = np.isneginf(ref)
    if clean:
        inf_gpu = np.isneginf(gpu)
        bad = inf_gpu != inf_ref
        assert not bad.any(), (f"{what}: -inf mask differs at {int(bad.sum())} entries, "
                               f"first {np.argwhere(bad)[:5].tolist()}")
    fin = ~inf_ref
    g, r, b = gpu[fin], ref[fin], bound[fin]
    assert np.isfinite(g).all(), f"{what}: non-finite value in range"
    if g.size:
        ratio = np.abs(g - r) / b
        k = int(np.argmax(ratio))
        log(f"   {what}: {g.size} in-range entries, max |gpu-ref|/bound = {ratio[k]:.3g}")
        assert ratio[k] <= 1.0, (f"{what}: |gpu-ref|/bound = {ratio[k]:.3g} "
                                 f"(gpu {g[k]!r}, ref {r[k]!r}, bound {b[k]!r})")
        return float(ratio.max())
    return 0.0


def assert_mask_on_device(out, k_start, k_end, skv, rows_per_chunk=256):
    """Full -inf mask check of a dense clean output on the device.

    Expected ranges come from the oracle's clamp; torch only compares."""
    s, e = oracle.row_ranges(k_start, k_end, skv)
    S = torch.from_numpy(s).to(out.device)
    E = torch.from_numpy(e).to(out.device)
    cols = torch.arange(skv, device=out.device)
    for r0 in range(0, out.shape[0], rows_per_chunk):
        r1 = min(r0 + rows_per_chunk, out.shape[0])
        valid = (cols[None, :] >= S[r0:r1, None]) & (cols[None, :] < E[r0:r1, None])
        chunk = out[r0:r1, :skv]
        assert torch.equal(torch.isneginf(chunk), ~valid), f"mask differs in rows [{r0}, {r1})"
        assert bool(torch.isfinite(chunk[valid]).all()), f"non-finite in range, rows [{r0}, {r1})"


def run_dense(case, clean=True, out=None):
    d = dense_on_device(case)
    import mqa_logits_amd as mq
    return mq.mqa_logits(d["fmt"], d["q"], d["q_sf"], d["kv"], d["kv_sf"], d["kv_scale"],
                         d["weights"], d["k_start"], d["k_end"], clean_logits=clean, out=out)


# ---------------------------------------------------------------------------
# The error class of the default precision (matrix-core grouped summation)
# ---------------------------------------------------------------------------
#
# In MQA_PRECISION_DEFAULT every aligned group of 8 fp8 products along D is
# summed after each product is truncated toward zero to a multiple of
# 2^(E - 13), E the exponent of the group's largest product (measured on the
# device).  The error of one dot is then below 7 * 2^(E - 13) per group <=
# 2^-10.19 * sum_d |q_d kv_d|, so with S = sum_h |w_h s_j| sum_d |q_hd kv_jd|
# the weighted head sum is off by less than about 2^-10.1 * S.  With H = 64 the
# linear half of ReLU comes from q' = sum_h (w_h / 2) q_h rounded to four e4m3
# pieces per 32-element block, which keeps about 16 bits below the block's
# largest |q'|: that adds at most 2^-15 * |s_j| sum_b max_{d in b} |q'_d|
# sum_{d in b} |kv_jd|.  The class bound below doubles the first term.

def default_class_bound(fmt, Q, K, kvs, w, lin):
    """Q [r, H, D], K [c, D] decoded (block scales applied), kvs [c], w [r, H]
    -> extra tolerance [r, c] of the default precision on top of the literal
    bound."""
    S = np.einsum("rh,rhc->rc", np.abs(w), np.abs(Q) @ np.abs(K).T) * np.abs(kvs)[None, :]
    extra = 2.0 ** -9 * S
    if lin:
        qp = np.einsum("rh,rhd->rd", w / 2.0, Q)                 # [r, D]
        nb = Q.shape[-1] // 32
        m = np.abs(qp).reshape(qp.shape[0], nb, 32).max(-1)      # [r, nb]
        ksum = np.abs(K).reshape(K.shape[0], nb, 32).sum(-1)     # [c, nb]
        extra = extra + 2.0 ** -15 * (m @ ksum.T) * np.abs(kvs)[None, :]
    return extra


def dense_class_bound(case, lin):
    Q = oracle.codecs.decode(case.fmt, case.q, case.q_sf)
    K = oracle.codecs.decode(case.fmt, case.kv, case.kv_sf)
    kvs = (np.ones(case.skv) if case.kv_scale is None
           else case.kv_scale.astype(np.float64))
    return default_class_bound(case.fmt, Q, K, kvs, case.weights.astype(np.float64), lin)


# ---------------------------------------------------------------------------
# Full rows of the large workloads: the oracle over row blocks on a thread
# pool (numpy releases the GIL in its matrix products and ufuncs), BLAS held
# to one thread per worker; each block is compared as it arrives.
# ---------------------------------------------------------------------------

def oracle_workers():
    import os
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def assert_rows_close(got_rows, case, rows, what, row_block=4):
    """got_rows: float32 [len(rows), Skv] from the GPU; rows: their indices.
    Runs oracle.dense_logits on blocks of row_block rows in parallel and checks
    every entry (mask bit-exact, values within the bound).  Returns the
    largest |gpu - ref| / bound."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    rows = np.asarray(rows, dtype=np.int64)
    starts = list(range(0, rows.size, row_block))

    def one(b0):
        r = rows[b0:b0 + row_block]
        ref, bound = oracle.dense_logits(*case.args(), rows=r, row_block=row_block)
        g = np.asarray(got_rows[b0:b0 + r.size], dtype=np.float64)
        inf_ref = np.isneginf(ref)
        if not np.array_equal(np.isneginf(g), inf_ref):
            bad = np.argwhere(np.isneginf(g) != inf_ref)[:3]
            return ("mask", int(r[0]), bad.tolist())
        fin = ~inf_ref
        if not np.isfinite(g[fin]).all():
            return ("nonfinite", int(r[0]), None)
        if not fin.any():
            return ("ok", 0.0, None)
        ratio = np.abs(g[fin] - ref[fin]) / bound[fin]
        return ("ok", float(ratio.max()), None)

    worst = 0.0
    with threadpool_limits(limits=1), ThreadPoolExecutor(oracle_workers()) as ex:
        for kind, val, extra in ex.map(one, starts):
            assert kind != "mask", f"{what}: -inf mask differs in the block at row {val}: {extra}"
            assert kind != "nonfinite", f"{what}: non-finite value in range near row {val}"
            worst = max(worst, val)
    log(f"   {what}: {rows.size} full rows, max |gpu-ref|/bound = {worst:.3g}")
    assert worst <= 1.0, f"{what}: |gpu-ref|/bound = {worst:.3g}"
    return worst
