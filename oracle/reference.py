"""float64 reference for dense, compressed and paged weighted MQA logits.

Test infrastructure (see the package header).

The quantity ([P1] "Core Architecture Components", Math Warp Reduction: after
the Q.KV^T product the scores go through ReLU, are multiplied by per-head
weights and are summed over heads; [P1] FAQ on quantization scales: a per-token
KV scale enters the score):

    logits[i, j] = sum_h w[i, h] * max(0, kv_scale[j] * <q[i, h, :], kv[j, :]>)

for j in the row's key range and -inf elsewhere ([P4] Description: a
clean_logits=True call writes negative infinity outside each row's range; the
reproducer checks that exactly the columns j >= ends[i] are -inf and that every
in-range entry of an all-zero problem is 0).  The KV scale multiplies the dot
product *inside* the ReLU, literally; for MX formats there is no per-token
scale (it is 1) and the block scales are part of the decoded values.

Readings taken where the pages leave a point open (each is listed in the design
notes as well):
  * ranges are half-open [k_start, k_end) ([P1] "Compressed Logits" bullet and
    Summary; [P4] reproducer compares cols < ends); they are clamped to
    s = clamp(k_start, 0, Skv), e = clamp(k_end, s, Skv), so e <= s is an empty
    row;
  * compressed rows hold only [s, e) of each row ([P1] "Compressed Logits"),
    packed one after another: row i starts at row_offsets[i], the exclusive
    prefix sum of the row lengths;
  * paged: query token t of sequence b is row b*next_n + t, its keys are the
    first ctx_b - next_n + t + 1 tokens of the sequence, and logical token j
    lives at slot j % block_size of physical block block_table[b, j // bs]
    ([P1] "Implementing Paged MQA Logits Computation for Decoding":
    context_lens is the length after adding the new tokens; [P3] "12cb7c0":
    next_n query tokens per sequence, block_kv the physical block size).

Every dot product here is exact: e4m3 values are multiples of 2^-9 below 2^9,
so a product is a multiple of 2^-18 below 2^18 and a 128-term sum spans fewer
than 53 bits; MX scales in [2^-127, 2^127] only shift that window per block and
the block sums stay exact as long as a dot's terms span < 53 bits, which holds
for the scale ranges the workloads use.  The matmul order therefore cannot
change a dot.  The only roundings are the float64 products with the fp32 KV
scale and weights and the sum over heads.

The error bound returned with each value is the tolerance of the GPU check:
    bound[i, j] = 1e-4 * sum_h |w[i, h] * kv_scale[j] * <q, kv>| + 1e-6.
"""

import numpy as np

from .codecs import decode

TOL_REL = 1e-4
TOL_ABS = 1e-6


def row_ranges(k_start, k_end, skv):
    """Clamped half-open key range [s_i, e_i) of every row (int64 arrays)."""
    ks = np.asarray(k_start, dtype=np.int64)
    ke = np.asarray(k_end, dtype=np.int64)
    s = np.clip(ks, 0, skv)
    e = np.clip(ke, s, skv)
    return s, e


def _weighted_relu_sum(Sdot, w, kvs):
    """Sdot [r, H, c] exact dots, w [r, H], kvs [c] -> (value [r, c], bound [r, c])."""
    x = Sdot * kvs[None, None, :]                      # kv_scale * <q, kv>
    wx = w[:, :, None]
    val = (wx * np.maximum(x, 0.0)).sum(axis=1)          # sum_h w * ReLU(.)
    bound = TOL_REL * np.abs(wx * x).sum(axis=1) + TOL_ABS
    return val, bound


def _decoded_inputs(fmt, q, q_sf, kv, kv_sf, kv_scale):
    Q = decode(fmt, q, q_sf)                             # [Sq, H, D]
    K = decode(fmt, kv, kv_sf)                           # [Skv, D]
    if fmt == "fp8":
        kvs = np.asarray(kv_scale, dtype=np.float32).astype(np.float64)
    else:
        if kv_scale is not None:
            raise ValueError("MX formats carry no per-token kv_scale (it is 1)")
        kvs = np.ones(K.shape[0], dtype=np.float64)
    return Q, K, kvs


def dense_logits(fmt, q, q_sf, kv, kv_sf, kv_scale, weights, k_start, k_end,
                 rows=None, row_block=16):
    """Dense clean logits for the selected rows.

    Returns (ref, bound), float64 [len(rows), Skv]; ref is -inf outside each
    row's range and bound is 0 there.  rows defaults to every row.
    """
    Q, K, kvs = _decoded_inputs(fmt, q, q_sf, kv, kv_sf, kv_scale)
    w = np.asarray(weights, dtype=np.float32).astype(np.float64)
    sq, skv = Q.shape[0], K.shape[0]
    rows = np.arange(sq) if rows is None else np.asarray(rows, dtype=np.int64)
    s, e = row_ranges(k_start, k_end, skv)
    ref = np.full((rows.size, skv), -np.inf)
    bound = np.zeros((rows.size, skv))
    KT = K.T
    cols = np.arange(skv)
    for b0 in range(0, rows.size, row_block):
        r = rows[b0:b0 + row_block]
        Sdot = Q[r] @ KT                                 # [r, H, Skv], exact
        val, bnd = _weighted_relu_sum(Sdot, w[r], kvs)
        valid = (cols[None, :] >= s[r, None]) & (cols[None, :] < e[r, None])
        ref[b0:b0 + r.size] = np.where(valid, val, -np.inf)
        bound[b0:b0 + r.size] = np.where(valid, bnd, 0.0)
    return ref, bound


def dense_entries(fmt, q, q_sf, kv, kv_sf, kv_scale, weights, k_start, k_end,
                  rows, cols):
    """Selected entries (rows[k], cols[k]) of the dense clean logits.

    rows and cols are equal-length index arrays.  Returns (ref, bound) float64
    [len(rows)]; out-of-range entries are -inf with bound 0.  Used where a full
    row is too large for the CPU to finish in seconds.
    """
    Q, K, kvs = _decoded_inputs(fmt, q, q_sf, kv, kv_sf, kv_scale)
    w = np.asarray(weights, dtype=np.float32).astype(np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    s, e = row_ranges(k_start, k_end, K.shape[0])
    Sdot = np.einsum("khd,kd->kh", Q[rows], K[cols])     # exact dots
    x = Sdot * kvs[cols][:, None]
    val = (w[rows] * np.maximum(x, 0.0)).sum(axis=1)
    bnd = TOL_REL * np.abs(w[rows] * x).sum(axis=1) + TOL_ABS
    valid = (cols >= s[rows]) & (cols < e[rows])
    return np.where(valid, val, -np.inf), np.where(valid, bnd, 0.0)


def compressed_row_offsets(k_start, k_end, skv):
    """int64 [Sq+1]: row i of the packed output starts at offsets[i]."""
    s, e = row_ranges(k_start, k_end, skv)
    out = np.zeros(s.size + 1, dtype=np.int64)
    np.cumsum(e - s, out=out[1:])
    return out


def compressed_logits(fmt, q, q_sf, kv, kv_sf, kv_scale, weights, k_start, k_end,
                      row_block=16):
    """Packed logits: row i's valid span [s_i, e_i) stored at offsets[i].

    Returns (packed_ref, packed_bound, offsets).
    """
    skv = np.asarray(kv).shape[0]
    s, e = row_ranges(k_start, k_end, skv)
    off = compressed_row_offsets(k_start, k_end, skv)
    ref, bound = dense_logits(fmt, q, q_sf, kv, kv_sf, kv_scale, weights,
                              k_start, k_end, row_block=row_block)
    packed = np.empty(int(off[-1]))
    pbound = np.empty(int(off[-1]))
    for i in range(s.size):
        packed[off[i]:off[i + 1]] = ref[i, s[i]:e[i]]
        pbound[off[i]:off[i + 1]] = bound[i, s[i]:e[i]]
    return packed, pbound, off


def paged_row_ranges(context_lens, next_n, max_context_len):
    """Key range [0, e) of row b*next_n + t: e = ctx_b - next_n + t + 1,
    clamped to [0, min(ctx_b, max_context_len)]."""
    ctx = np.asarray(context_lens, dtype=np.int64)
    t = np.arange(next_n, dtype=np.int64)
    e = ctx[:, None] - next_n + t[None, :] + 1
    hi = np.minimum(ctx, max_context_len)[:, None]
    e = np.clip(e, 0, hi).reshape(-1)
    return np.zeros_like(e), e


def gather_paged_kv(kv_pool, kv_scale_pool, block_table, b, length, block_size):
    """Logical tokens [0, length) of sequence b, gathered through the block table."""
    j = np.arange(length)
    blk = np.asarray(block_table)[b, j // block_size]
    slot = j % block_size
    kv = np.asarray(kv_pool)[blk, slot]
    kvs = None if kv_scale_pool is None else np.asarray(kv_scale_pool)[blk, slot]
    return kv, kvs


def paged_logits(fmt, q, q_sf, kv_pool, kv_sf_pool, kv_scale_pool, weights,
                 context_lens, block_table, next_n, block_size, max_context_len):
    """Paged decode logits: (ref, bound) float64 [batch*next_n, max_context_len]."""
    ctx = np.asarray(context_lens, dtype=np.int64)
    batch = ctx.size
    _, e = paged_row_ranges(ctx, next_n, max_context_len)
    ref = np.full((batch * next_n, max_context_len), -np.inf)
    bound = np.zeros_like(ref)
    for b in range(batch):
        length = int(min(ctx[b], max_context_len))
        kv, kvs = gather_paged_kv(kv_pool, kv_scale_pool, block_table, b, length, block_size)
        kv_sf = None
        if kv_sf_pool is not None:
            kv_sf, _ = gather_paged_kv(kv_sf_pool, None, block_table, b, length, block_size)
        r = slice(b * next_n, (b + 1) * next_n)
        sub_ref, sub_bound = dense_logits(
            fmt, q[r], None if q_sf is None else q_sf[r], kv, kv_sf, kvs,
            weights[r], np.zeros(next_n, np.int64), e[r])
        ref[r, :length] = sub_ref
        bound[r, :length] = sub_bound
    return ref, bound
