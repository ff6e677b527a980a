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
