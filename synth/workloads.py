"""Seeded generators for the MQA-logits workloads.

Random streams: numpy Generator(PCG64) seeded with [case_seed, tensor_id] so
every tensor of a case has its own reproducible stream:
    q=0, kv=1, kv_scale=2, weights=3, context_lens=4, block permutation=5,
    q block scales=6, kv block scales=7, sampled rows=8.

Value recipes (the shapes and distributions of the workloads the pages time):
  * FP8 Q and KV: N(0, 1), clipped to +-448, rounded to nearest-even e4m3fn;
  * kv_scale: fp32 U(0.5, 2);  weights: fp32 N(0, 1/H) (std 1/sqrt(H));
  * MX: per block of 32 elements an exponent e ~ U{-2..2} (scale byte 127+e)
    and elements round_to_nearest_even_saturating(x * 2^-e), x ~ N(0, 1),
    saturating at +-448 (e4m3) or +-6 (e2m1);
  * paged: context lengths U{lo..hi} inclusive, block table rows taken from
    one random permutation of the physical block pool.
"""

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

E4M3_MAX = 448.0
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])

TENSOR_IDS = dict(q=0, kv=1, kv_scale=2, weights=3, context_lens=4, perm=5,
                  q_sf=6, kv_sf=7, rows=8, pairs=10)


def stream(seed, name):
    return np.random.default_rng([int(seed), TENSOR_IDS[name]])


# --------------------------------------------------------------------------
# encoders (input preparation only)
# --------------------------------------------------------------------------

def encode_bf16(x):
    """float32 array -> uint16 bfloat16 bit patterns, nearest with ties to
    even (finite inputs).  bf16 weights are an input format; the value both
    sides see is decode_bf16 of these bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def decode_bf16(bits):
    """uint16 bfloat16 bit patterns -> their exact float32 values."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def encode_e4m3(x):
    """float array -> uint8 e4m3fn codes, clipped to +-448, ties to even."""
    x = np.clip(np.asarray(x, dtype=np.float32), -E4M3_MAX, E4M3_MAX)
    t = torch.from_numpy(np.ascontiguousarray(x)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def encode_e2m1(x):
    """float array -> uint8 e2m1 nibbles (0..15), saturating at 6, ties to even."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 6.0)
    hi = np.clip(np.searchsorted(E2M1_GRID, a, side="left"), 0, 7)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - E2M1_GRID[lo]
    d_hi = E2M1_GRID[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return code | np.where(np.signbit(x), 0x8, 0).astype(np.uint8)


def pack_e2m1(nibbles):
    """[..., 2n] nibbles -> [..., n] bytes; element 2k in the low nibble."""
    nibbles = np.asarray(nibbles, dtype=np.uint8)
    return (nibbles[..., 0::2] | (nibbles[..., 1::2] << 4)).astype(np.uint8)


def _fp8_values(rng, shape):
    return encode_e4m3(rng.standard_normal(shape, dtype=np.float32))


def _mx_values(fmt, rng_val, rng_sf, shape):
    """shape = (..., D) -> (codes, scale bytes [..., D/32])."""
    *lead, d = shape
    nb = d // 32
    e = rng_sf.integers(-2, 3, size=(*lead, nb))
    x = rng_val.standard_normal(shape, dtype=np.float32).astype(np.float64)
    x = x * np.repeat(2.0 ** (-e), 32, axis=-1)
    if fmt == "mxfp8":
        codes = encode_e4m3(x)
    else:
        codes = pack_e2m1(encode_e2m1(x))
    return codes, (127 + e).astype(np.uint8)


# --------------------------------------------------------------------------
# dense / compressed cases
# --------------------------------------------------------------------------

@dataclass
class DenseCase:
    fmt: str
    sq: int
    skv: int
    h: int
    d: int
    q: np.ndarray                      # uint8 [Sq, H, D] (fp4: [Sq, H, D/2])
    q_sf: Optional[np.ndarray]         # uint8 [Sq, H, D/32] or None
    kv: np.ndarray                     # uint8 [Skv, D]   (fp4: [Skv, D/2])
    kv_sf: Optional[np.ndarray]        # uint8 [Skv, D/32] or None
    kv_scale: Optional[np.ndarray]     # float32 [Skv] (fp8 only)
    weights: np.ndarray                # float32 [Sq, H]
    k_start: np.ndarray                # int32 [Sq]
    k_end: np.ndarray                  # int32 [Sq]
    seed: int = 0
    name: str = ""

    def args(self):
        """Positional inputs shared by the oracle and the GPU binding."""
        return (self.fmt, self.q, self.q_sf, self.kv, self.kv_sf, self.kv_scale,
                self.weights, self.k_start, self.k_end)


def dense_case(sq, skv, h, d, fmt="fp8", seed=0, k_start=None, k_end=None,
               zero=False, name=""):
    """A dense problem; ranges default to the full row [0, Skv)."""
    if fmt not in ("fp8", "mxfp8", "mxfp4"):
        raise ValueError(fmt)
    q_sf = kv_sf = kv_scale = None
    if fmt == "fp8":
        q = _fp8_values(stream(seed, "q"), (sq, h, d))
        kv = _fp8_values(stream(seed, "kv"), (skv, d))
        kv_scale = stream(seed, "kv_scale").uniform(0.5, 2.0, skv).astype(np.float32)
    else:
        q, q_sf = _mx_values(fmt, stream(seed, "q"), stream(seed, "q_sf"), (sq, h, d))
        kv, kv_sf = _mx_values(fmt, stream(seed, "kv"), stream(seed, "kv_sf"), (skv, d))
    weights = (stream(seed, "weights").standard_normal((sq, h)) / np.sqrt(h)).astype(np.float32)
    if zero:
        q[...] = 0
        kv[...] = 0
        weights[...] = 0
        if q_sf is not None:
            q_sf[...] = 127
            kv_sf[...] = 127
    if k_start is None:
        k_start = np.zeros(sq, np.int32)
    if k_end is None:
        k_end = np.full(sq, skv, np.int32)
    return DenseCase(fmt, sq, skv, h, d, q, q_sf, kv, kv_sf, kv_scale, weights,
                     np.asarray(k_start, np.int32), np.asarray(k_end, np.int32),
                     seed, name)


# --------------------------------------------------------------------------
# paged cases
# --------------------------------------------------------------------------

POISON_FP8 = 0x7F        # an e4m3fn NaN code: any read of an unused block shows


@dataclass
class PagedCase:
    fmt: str
    batch: int
    next_n: int
    h: int
    d: int
    block_size: int
    num_blocks: int
    max_context_len: int
    q: np.ndarray                      # uint8 [batch*next_n, H, D]
    q_sf: Optional[np.ndarray]
    kv_pool: np.ndarray                # uint8 [num_blocks, block_size, D]
    kv_sf_pool: Optional[np.ndarray]   # uint8 [num_blocks, block_size, D/32]
    kv_scale_pool: Optional[np.ndarray]  # float32 [num_blocks, block_size]
    weights: np.ndarray                # float32 [batch*next_n, H]
    context_lens: np.ndarray           # int32 [batch]
    block_table: np.ndarray            # int32 [batch, max_blocks_per_seq]
    seed: int = 0
    name: str = ""

    def args(self):
        return (self.fmt, self.q, self.q_sf, self.kv_pool, self.kv_sf_pool,
                self.kv_scale_pool, self.weights, self.context_lens,
                self.block_table, self.next_n, self.block_size,
                self.max_context_len)


def paged_case(batch, next_n, h, d, block_size, num_blocks, ctx_lo, ctx_hi,
               max_context_len, fmt="fp8", seed=0, context_lens=None,
               poison_unused=True, name=""):
    """A paged decode problem.

    Blocks that no sequence reads are filled with NaN codes (and NaN scales) so
    that a wrong block index shows up as a non-finite output.
    """
    mbps = -(-max_context_len // block_size)
    if context_lens is None:
        context_lens = stream(seed, "context_lens").integers(ctx_lo, ctx_hi + 1, size=batch)
    context_lens = np.asarray(context_lens, dtype=np.int32)
    perm = stream(seed, "perm").permutation(num_blocks).astype(np.int32)
    flat = (np.arange(batch)[:, None] * mbps + np.arange(mbps)[None, :]) % num_blocks
    block_table = perm[flat].astype(np.int32)

    n_used = -(-np.minimum(context_lens.astype(np.int64), max_context_len) // block_size)
    used = np.zeros(num_blocks, dtype=bool)
    for b in range(batch):
        used[block_table[b, :n_used[b]]] = True
    used_ids = np.nonzero(used)[0]

    kb = d // 2 if fmt == "mxfp4" else d
    kv_pool = np.full((num_blocks, block_size, kb), POISON_FP8 if poison_unused else 0, np.uint8)
    kv_sf_pool = kv_scale_pool = q_sf = None
    if fmt == "fp8":
        kv_pool[used_ids] = _fp8_values(stream(seed, "kv"), (used_ids.size, block_size, d))
        kv_scale_pool = np.full((num_blocks, block_size),
                                np.nan if poison_unused else 1.0, np.float32)
        kv_scale_pool[used_ids] = stream(seed, "kv_scale").uniform(
            0.5, 2.0, (used_ids.size, block_size)).astype(np.float32)
        q = _fp8_values(stream(seed, "q"), (batch * next_n, h, d))
    else:
        kv_sf_pool = np.full((num_blocks, block_size, d // 32), 127, np.uint8)
        codes, sf = _mx_values(fmt, stream(seed, "kv"), stream(seed, "kv_sf"),
                               (used_ids.size, block_size, d))
        kv_pool[used_ids] = codes
        kv_sf_pool[used_ids] = sf
        if poison_unused:
            kv_sf_pool[~used] = 0xFF          # e8m0 NaN
        q, q_sf = _mx_values(fmt, stream(seed, "q"), stream(seed, "q_sf"),
                             (batch * next_n, h, d))
    weights = (stream(seed, "weights").standard_normal((batch * next_n, h)) / np.sqrt(h)).astype(np.float32)
    return PagedCase(fmt, batch, next_n, h, d, block_size, num_blocks, max_context_len,
                     q, q_sf, kv_pool, kv_sf_pool, kv_scale_pool, weights,
                     context_lens, block_table, seed, name)


# --------------------------------------------------------------------------
# cancelling dot products
# --------------------------------------------------------------------------
#
# Inputs whose dots cancel: in every aligned group of 8 elements along D two
# fixed positions carry +CANCEL_BIG and -CANCEL_BIG in Q and one equal value
# in KV, so their products cancel exactly and the dot is the sum of the six
# small products of each group.  Values are chosen so that every partial sum
# of the products is a multiple of 2^-9 below 2^14 in magnitude (at most 23
# significant bits): exact in fp32 in any order.
#   Q: the pair, and smalls +-m * 2^-5 with m in {1, 1.125, .., 1.875};
#   KV: +-1 or +-2 per element, the pair's two elements equal;
#   MX: q block scales 2^-1 or 2^0, kv block scales 2^0 or 2^1.

CANCEL_BIG = 128.0


def cancel_pairs(seed, d):
    """[D/8, 2]: the two positions of each group's cancelling pair."""
    rng = stream(seed, "pairs")
    return np.stack([rng.choice(8, 2, replace=False) for _ in range(d // 8)])


def _cancel_q(rng, shape, pairs):
    d = shape[-1]
    x = rng.choice([-1.0, 1.0], size=shape) * (1.0 + rng.integers(0, 8, size=shape) / 8.0) / 32.0
    g = np.arange(d // 8) * 8
    x[..., g + pairs[:, 0]] = CANCEL_BIG
    x[..., g + pairs[:, 1]] = -CANCEL_BIG
    return encode_e4m3(x)


def _cancel_kv(rng, shape, pairs):
    d = shape[-1]
    x = rng.choice([-2.0, -1.0, 1.0, 2.0], size=shape)
    g = np.arange(d // 8) * 8
    x[..., g + pairs[:, 1]] = x[..., g + pairs[:, 0]]
    return encode_e4m3(x)


def cancelling_dense_case(sq, skv, h, d, fmt="fp8", seed=0, k_start=None, k_end=None):
    """dense_case with cancelling Q and KV codes (fp8 or mxfp8)."""
    if fmt not in ("fp8", "mxfp8"):
        raise ValueError(fmt)
    case = dense_case(sq, skv, h, d, fmt, seed, k_start, k_end,
                      name=f"cancelling_{fmt}_h{h}_d{d}")
    pairs = cancel_pairs(seed, d)
    case.q = _cancel_q(stream(seed, "q"), (sq, h, d), pairs)
    case.kv = _cancel_kv(stream(seed, "kv"), (skv, d), pairs)
    if fmt == "mxfp8":
        case.q_sf = (126 + stream(seed, "q_sf").integers(0, 2, (sq, h, d // 32))).astype(np.uint8)
        case.kv_sf = (127 + stream(seed, "kv_sf").integers(0, 2, (skv, d // 32))).astype(np.uint8)
    return case


def cancelling_paged_case(batch, next_n, h, d, block_size, num_blocks, ctx_lo, ctx_hi,
                          max_context_len, fmt="fp8", seed=0):
    """paged_case with cancelling Q and KV codes in the blocks it reads."""
    if fmt not in ("fp8", "mxfp8"):
        raise ValueError(fmt)
    case = paged_case(batch, next_n, h, d, block_size, num_blocks, ctx_lo, ctx_hi,
                      max_context_len, fmt, seed, name=f"cancelling_paged_{fmt}_h{h}_d{d}")
    pairs = cancel_pairs(seed, d)
    case.q = _cancel_q(stream(seed, "q"), case.q.shape, pairs)
    n_used = -(-np.minimum(case.context_lens.astype(np.int64), max_context_len) // block_size)
    used = np.unique(np.concatenate([case.block_table[b, :n_used[b]] for b in range(batch)]))
    case.kv_pool[used] = _cancel_kv(stream(seed, "kv"), (used.size, block_size, d), pairs)
    if fmt == "mxfp8":
        case.q_sf = (126 + stream(seed, "q_sf").integers(0, 2, case.q_sf.shape)).astype(np.uint8)
        case.kv_sf_pool[used] = (127 + stream(seed, "kv_sf").integers(
            0, 2, (used.size, block_size, d // 32))).astype(np.uint8)
    return case


# --------------------------------------------------------------------------
# the five named workloads
# --------------------------------------------------------------------------

WORKLOAD_NAMES = {
    0: "dense_tiny_sq256_skv1024_h16_d64_fp8",
    1: "dense_prefill_sq2048_skv32768_h64_d128_fp8",
    2: "compressed_sq2048_skv4096_h32_d64_fp8",
    3: "paged_decode_b64_nextn4_h64_d128_bs64_fp8",
    4: "dense_mx_sq8192_skv65536_h64_d128",
}


def workload_case(idx, fmt=None, zero=False):
    """The five workloads, seeded with 1000 + idx.  idx 4 takes fmt
    'mxfp8' (default) or 'mxfp4'; idx 1 and 3 take 'fp8' (default), 'mxfp8'
    or 'mxfp4' (idx 1: the shape the pages time their MX kernels on).  zero: the dense
    workloads with all-zero Q, KV and weights and unit MX scales (the pages'
    timing workload)."""
    seed = 1000 + idx
    if zero and idx == 3:
        raise ValueError("the paged workload has no all-zero variant")
    if idx == 0:
        sq, skv = 256, 1024
        return dense_case(sq, skv, 16, 64, "fp8", seed, k_end=skv - sq + np.arange(sq) + 1,
                          zero=zero, name=WORKLOAD_NAMES[0])
    if idx == 1:
        fmt = fmt or "fp8"
        sq, skv = 2048, 32768
        name = WORKLOAD_NAMES[1] if fmt == "fp8" else WORKLOAD_NAMES[1].replace("_fp8", "_" + fmt)
        return dense_case(sq, skv, 64, 128, fmt, seed, k_end=skv - sq + np.arange(sq),
                          zero=zero, name=name)
    if idx == 2:
        sq, skv = 2048, 4096
        return dense_case(sq, skv, 32, 64, "fp8", seed, k_start=np.arange(sq),
                          k_end=np.full(sq, skv), zero=zero, name=WORKLOAD_NAMES[2])
    if idx == 3:
        fmt = fmt or "fp8"
        name = WORKLOAD_NAMES[3] if fmt == "fp8" else WORKLOAD_NAMES[3].replace("_fp8", "_" + fmt)
        return paged_case(64, 4, 64, 128, 64, 36000, 1024, 32768, 32768, fmt, seed, name=name)
    if idx == 4:
        fmt = fmt or "mxfp8"
        sq, skv = 8192, 65536
        return dense_case(sq, skv, 64, 128, fmt, seed, k_end=skv - sq + np.arange(sq),
                          zero=zero, name=WORKLOAD_NAMES[4] + "_" + fmt)
    raise ValueError(idx)


def topk_logits(sq, skv, seed, ties=True, ranges=True):
    """Synthetic logits rows for the top-k selection: N(0, 1) values (on a
    1/16 grid when `ties`, so equal values are common), about 5% -inf and 2%
    signed zeros inside the rows, -inf outside the ranges.  Returns
    (logits float32 [Sq, Skv], k_start, k_end) with the ranges None when
    `ranges` is false; ranges mix full, empty, short and shifted rows."""
    rng = np.random.default_rng([int(seed), 9])
    x = rng.standard_normal((sq, skv))
    if ties:
        x = np.round(x * 16) / 16
    x[rng.random((sq, skv)) < 0.05] = -np.inf
    z = rng.random((sq, skv)) < 0.02
    x[z] = np.where(rng.random(int(z.sum())) < 0.5, 0.0, -0.0)
    x = x.astype(np.float32)
    if not ranges:
        return x, None, None
    ks = rng.integers(-10, skv, sq)
    ke = ks + rng.integers(-20, skv + 20, sq)
    if sq >= 4:
        ks[:4] = [0, 5, skv // 2, 0]
        ke[:4] = [skv, 5, skv // 2 + 3, skv + 100]      # full, empty, short, past the end
    cols = np.arange(skv)[None, :]
    s = np.clip(ks, 0, skv)[:, None]
    e = np.clip(ke, np.clip(ks, 0, skv), skv)[:, None]
    x[(cols < s) | (cols >= e)] = -np.inf
    return x, ks.astype(np.int32), ke.astype(np.int32)


def sampled_rows(seed, sq, n):
    """n distinct rows in [0, Sq), always including 0 and Sq-1, sorted."""
    if n >= sq:
        return np.arange(sq)
    rest = stream(seed, "rows").choice(np.arange(1, sq - 1), size=n - 2, replace=False)
    return np.sort(np.concatenate([[0, sq - 1], rest])).astype(np.int64)
