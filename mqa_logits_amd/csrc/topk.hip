// Top-k selection over logits rows for gfx950: the consumer of the logits in
// sparse attention ("FlashMLA", flash_mla_with_kvcache's optional `indices`
// of shape (batch, seq_len_q, topk), -1 for invalid entries; the top-k
// sparsity parameter of get_mla_metadata).
//
// Row i's candidates are its columns j in [s_i, e_i) whose logit is not -inf.
// The selection is the topk largest candidates, equal values ranked by
// smaller column first, so it is unique; it is written in ascending column
// order and padded with -1 when a row has fewer than topk candidates.
//
// One block of 1024 threads per row.  Logits map to order-preserving 32-bit
// keys (sign-magnitude to two's-complement order); the selection is the
// topk-th largest key K and how many keys equal to K to keep.  Rows of up to
// 65536 columns are held in registers (topk_reg_kernel below: a sampled
// threshold narrows the row to a short LDS list first).  Longer rows stream
// (topk_stream_kernel), with a radix select over the keys (11 + 11 + 10
// bits, one LDS histogram per level):
//   * A first pass over the row builds the top-11-bit histogram: the bin B of
//     the topk-th key, the count above it and the count in it.
//   * When both counts fit in LDS (the usual case) a second pass copies, in
//     column order, the columns above B and the (key, column) pairs in B to
//     LDS; the last two levels, the choice of B's keys and the merge of the
//     two column-ordered lists into the output run in LDS.  Two passes over
//     the row in all.
//   * Otherwise every level is a pass over the row, and a last pass writes
//     the selected columns in column order with a block-wide prefix count of
//     (keys > K, keys == K).
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace mqa {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWaveLanes;
constexpr uint32_t kKeyNegInf = 0x007FFFFFu;       // key of -inf: not a candidate
constexpr uint32_t kBitsNegInf = 0xFF800000u;      // fp32 bits of -inf

// Order-preserving key of an fp32 bit pattern: larger float, larger key.
__device__ __forceinline__ uint32_t order_key(uint32_t bits) {
  return (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
}

template <int IN>
struct TopkRow {
  Rsrc r;                                 // the row's Skv elements
  int s;                                  // first column of the range (element offset)
  int last;                               // the buffer's last column, relative to s
  // Key of column s + c (c relative to the range start).  The caller keeps
  // c inside the range.
  __device__ __forceinline__ uint32_t key(int c) const {
    uint32_t bits;
    if constexpr (IN == kBF16) {
      bits = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, 2 * (s + c), 0, 0) << 16;
    } else {
      bits = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, 4 * (s + c), 0, 0);
    }
    return order_key(bits);
  }
  // fp32 bit patterns of columns s + c .. s + c + 3 (one 8- or 16-byte load);
  // columns at or past n (the range end, relative) read as -inf unless the
  // caller knows all four are in range (`full`).
  __device__ __forceinline__ void bits4(int c, int n, bool full, uint32_t (&b)[4]) const {
    uint32_t bits[4];
    if constexpr (IN == kBF16) {
      typedef int v2i __attribute__((ext_vector_type(2)));
      const v2i w = __builtin_amdgcn_raw_buffer_load_b64(r, 2 * (s + c), 0, 0);
      bits[0] = (uint32_t)w[0] << 16;
      bits[1] = (uint32_t)w[0] & 0xffff0000u;
      bits[2] = (uint32_t)w[1] << 16;
      bits[3] = (uint32_t)w[1] & 0xffff0000u;
      // The buffer checks each 4-byte half of the load against its end and
      // reads a half that crosses it as zero: when the buffer's last column
      // (an odd end) opens a half, that column is read on its own.
      const int lu = last - c;
      if (lu == 0 || lu == 2)
        bits[lu] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, 2 * (s + c + lu), 0, 0) << 16;
    } else {
      typedef int v4i __attribute__((ext_vector_type(4)));
      const v4i w = __builtin_amdgcn_raw_buffer_load_b128(r, 4 * (s + c), 0, 0);
      for (int u = 0; u < 4; ++u) bits[u] = (uint32_t)w[u];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) b[u] = full || c + u < n ? bits[u] : kBitsNegInf;
  }
};

// ---- wave-level scans and reductions ----------------------------------------
// Inclusive scans over the wave with DPP moves (ALU latency, no LDS round
// trips): shifts by 1, 2, 4 and 8 lanes within each row of 16, then row 0's
// and row 1's last lanes broadcast to the rows after them.  `id` is the
// operation's identity, which lanes without a source contribute.
template <class Op>
__device__ __forceinline__ uint32_t wave_scan_u32(uint32_t x, uint32_t id, Op op) {
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x111, 0xf, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x112, 0xf, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x114, 0xf, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x118, 0xf, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x142, 0xa, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x143, 0xc, 0xf, false));
  return x;
}
struct OpAdd {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; }
};
struct OpMax {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return max(a, b); }
};
struct OpMin {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return min(a, b); }
};
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_scan_u32(v, 0u, OpMax{}), kWaveLanes - 1);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_scan_u32(v, ~0u, OpMin{}), kWaveLanes - 1);
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_scan_u32(v, 0u, OpAdd{}), kWaveLanes - 1);
}

// Inclusive sum over the wave; a 64-bit value is a pair of 32-bit counts
// (high, low) that never carry into each other, scanned as two.  Every lane
// of the wave takes part.
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t x) {
  return wave_scan_u32(x, 0u, OpAdd{});
}
__device__ __forceinline__ uint64_t wave_incl_sum(uint64_t x) {
  return ((uint64_t)wave_scan_u32((uint32_t)(x >> 32), 0u, OpAdd{}) << 32) |
         wave_scan_u32((uint32_t)x, 0u, OpAdd{});
}

// Exclusive prefix sum over the block (thread order) of a per-thread value;
// *total receives the block total.  Every thread must call it.
template <class T>
__device__ __forceinline__ T block_exclusive_scan(T v, T* wave_sums, T* total) {
  const int lane = threadIdx.x & (kWaveLanes - 1);
  const int wave = threadIdx.x >> 6;
  const T x = wave_incl_sum(v);
  if (lane == kWaveLanes - 1) wave_sums[wave] = x;
  __syncthreads();
  if (wave == 0) {
    T w = lane < kTopkWaves ? wave_sums[lane] : T(0);
    w = wave_incl_sum(w);
    if (lane < kTopkWaves) wave_sums[lane] = w;             // inclusive per wave
  }
  __syncthreads();
  const T before = wave > 0 ? wave_sums[wave - 1] : T(0);
  *total = wave_sums[kTopkWaves - 1];
  __syncthreads();                                          // wave_sums reusable after this
  return before + x - v;
}

constexpr int kTopkCap = 4 * kTopkThreads;   // LDS list capacity of the two-pass path


// 2048 bins and a spare slot; the stride puts a bin's four copies in four
// different LDS banks (2064 = 16 mod 64)
constexpr int kHistStride = 2048 + 16;

struct TopkShared {
  alignas(16) uint32_t hist[kHistStride];   // 16-byte rows: read as 4-bin vectors
  uint64_t wave_sums64[kTopkWaves];
  uint32_t wave_sums32[kTopkWaves];
  uint32_t sel_bin, sel_above;
};

// The streaming kernel's column lists.
struct TopkLists {
  int32_t d_col[kTopkCap];    // columns above the first-level bin, in column order
  uint32_t b_key[kTopkCap];   // keys in that bin (column order), then the chosen columns
  int32_t b_col[kTopkCap];
};

// Elements of the ascending list a[0, n) below x.
__device__ __forceinline__ int count_below(const int32_t* a, int n, int32_t x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// One radix level over the histogram in sh.hist (nbins = 2048 or 1024, in
// descending bin order): the bin holding the need-th largest key and the
// number of keys in higher bins.
__device__ __forceinline__ void find_bin(TopkShared& sh, int nbins, uint32_t need) {
  const int t = threadIdx.x;
  const int per = nbins / kTopkThreads;                     // 2 or 1 bins per thread
  uint32_t local = 0;
  for (int k = 0; k < per; ++k) local += sh.hist[nbins - 1 - (per * t + k)];
  uint32_t total;
  uint32_t above = block_exclusive_scan<uint32_t>(local, sh.wave_sums32, &total);
  for (int k = 0; k < per; ++k) {
    const int b = nbins - 1 - (per * t + k);
    const uint32_t c = sh.hist[b];
    if (above < need && above + c >= need) {
      sh.sel_bin = (uint32_t)b;
      sh.sel_above = above;
    }
    above += c;
  }
  __syncthreads();
}

// One row of any length, read from memory once per level (the streaming
// selection); sh and ls are the block's LDS.  Every thread of the block calls it.
template <int IN>
__device__ void topk_stream_row(const TopkParams& p, int64_t row, TopkShared& sh, TopkLists& ls) {
  const int t = threadIdx.x;
  int s = 0, e = p.skv;
  if (p.k_start) {
    s = clampi(p.k_start[row], 0, p.skv);
    e = clampi(p.k_end[row], s, p.skv);
  }
  const int n = e - s;
  constexpr int kIB = IN == kBF16 ? 2 : 4;
  const TopkRow<IN> src{make_rsrc(static_cast<const char*>(p.logits) + row * p.stride * kIB,
                                  (uint32_t)(p.skv * kIB)),
                        s, p.skv - 1 - s};
  int32_t* out = p.indices + row * p.out_stride;

  // ---- first level over the row: histogram of the top 11 bits -------------
  constexpr int kShift[3] = {21, 10, 0};
  constexpr int kBins[3] = {2048, 2048, 1024};
  auto histogram_pass = [&](int lvl, uint32_t prefix, uint32_t mask) {
    for (int b = t; b < kBins[lvl]; b += kTopkThreads) sh.hist[b] = 0;
    __syncthreads();
    // four loads in flight per thread before their histogram updates
    for (int c = t; c < n; c += 4 * kTopkThreads) {
      uint32_t k[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        k[u] = c + u * kTopkThreads < n ? src.key(c + u * kTopkThreads) : kKeyNegInf;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (k[u] != kKeyNegInf && (k[u] & mask) == prefix)
          atomicAdd(&sh.hist[(k[u] >> kShift[lvl]) & (kBins[lvl] - 1)], 1u);
    }
    __syncthreads();
  };
  histogram_pass(0, 0u, 0u);
  uint32_t n_cand;
  {
    uint32_t local = 0;
    for (int b = t; b < 2048; b += kTopkThreads) local += sh.hist[b];
    block_exclusive_scan<uint32_t>(local, sh.wave_sums32, &n_cand);
  }
  const bool take_all = n_cand <= (uint32_t)p.topk;     // every candidate is selected
  uint32_t need = (uint32_t)p.topk;         // keys still to place at or below the prefix
  uint32_t prefix = 0, mask = 0;
  uint32_t n_above = 0, n_bin = 0;
  if (!take_all) {
    find_bin(sh, 2048, need);
    const uint32_t b1 = sh.sel_bin;
    n_above = sh.sel_above;
    n_bin = sh.hist[b1];
    need -= n_above;
    prefix = b1 << kShift[0];
    mask = 2047u << kShift[0];
    __syncthreads();                        // sel_* and hist read by all
  }

  if (!take_all && n_above <= (uint32_t)kTopkCap && n_bin <= (uint32_t)kTopkCap) {
    // ---- second pass: the columns above the bin and the bin's (key, column)
    // pairs, both in column order, into LDS ----------------------------------
    constexpr int kTile = 4 * kTopkThreads;
    uint64_t carry = 0;                     // (in bin << 32) | above, before the tile
    for (int c0 = 0; c0 < n; c0 += kTile) {
      const int c = c0 + 4 * t;
      uint32_t kk[4];
      uint32_t na = 0, nb = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        kk[u] = c + u < n ? src.key(c + u) : kKeyNegInf;
        const bool valid = kk[u] != kKeyNegInf;
        na += (valid && (kk[u] & mask) > prefix) ? 1u : 0u;
        nb += (valid && (kk[u] & mask) == prefix) ? 1u : 0u;
      }
      uint64_t tile_total;
      const uint64_t before = carry + block_exclusive_scan<uint64_t>(((uint64_t)nb << 32) | na,
                                                                     sh.wave_sums64, &tile_total);
      uint32_t ab = (uint32_t)before, bb = (uint32_t)(before >> 32);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool valid = kk[u] != kKeyNegInf;
        if (valid && (kk[u] & mask) > prefix) {
          if (ab < (uint32_t)kTopkCap) ls.d_col[ab] = s + c + u;
          ++ab;
        } else if (valid && (kk[u] & mask) == prefix) {
          if (bb < (uint32_t)kTopkCap) {
            ls.b_key[bb] = kk[u];
            ls.b_col[bb] = s + c + u;
          }
          ++bb;
        }
      }
      carry += tile_total;
    }
    __syncthreads();
    const int n_d = (int)n_above, n_b = (int)n_bin;

    // ---- levels 2 and 3 over the bin's keys in LDS --------------------------
#pragma unroll
    for (int lvl = 1; lvl < 3; ++lvl) {
      for (int b = t; b < kBins[lvl]; b += kTopkThreads) sh.hist[b] = 0;
      __syncthreads();
      for (int i = t; i < n_b; i += kTopkThreads) {
        const uint32_t k = ls.b_key[i];
        if ((k & mask) == prefix) atomicAdd(&sh.hist[(k >> kShift[lvl]) & (kBins[lvl] - 1)], 1u);
      }
      __syncthreads();
      find_bin(sh, kBins[lvl], need);
      need -= sh.sel_above;
      prefix |= sh.sel_bin << kShift[lvl];
      mask |= (uint32_t)(kBins[lvl] - 1) << kShift[lvl];
      __syncthreads();
    }
    const uint32_t K = prefix, need_eq = need;

    // ---- the bin's chosen columns, in column order, over its keys -----------
    uint32_t kk[4];
    int32_t cc[4];
    uint32_t g = 0, q = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = 4 * t + u;
      kk[u] = i < n_b ? ls.b_key[i] : 0u;
      cc[u] = i < n_b ? ls.b_col[i] : 0;
      g += (i < n_b && kk[u] > K) ? 1u : 0u;
      q += (i < n_b && kk[u] == K) ? 1u : 0u;
    }
    uint64_t total;
    const uint64_t before =
        block_exclusive_scan<uint64_t>(((uint64_t)q << 32) | g, sh.wave_sums64, &total);
    int32_t* chosen = reinterpret_cast<int32_t*>(ls.b_key);   // every key is in registers now
    const int n_c = (int)(p.topk - n_above);
    uint32_t gb = (uint32_t)before, qb = (uint32_t)(before >> 32);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = 4 * t + u;
      if (i < n_b && kk[u] > K) {
        const uint32_t pos = gb + min(qb, need_eq);
        if (pos < (uint32_t)kTopkCap) chosen[pos] = cc[u];
        ++gb;
      } else if (i < n_b && kk[u] == K) {
        if (qb < need_eq && gb + qb < (uint32_t)kTopkCap) chosen[gb + qb] = cc[u];
        ++qb;
      }
    }
    __syncthreads();

    // ---- merge the two ascending lists into the row's indices ----------------
    for (int i = t; i < n_d; i += kTopkThreads) {
      const int pos = i + count_below(chosen, n_c, ls.d_col[i]);
      if (pos < p.topk) out[pos] = ls.d_col[i];
    }
    for (int j = t; j < n_c; j += kTopkThreads) {
      const int pos = j + count_below(ls.d_col, n_d, chosen[j]);
      if (pos < p.topk) out[pos] = chosen[j];
    }
    return;
  }

  // ---- otherwise: levels 2 and 3 as passes over the row ---------------------
  if (!take_all) {
#pragma unroll
    for (int lvl = 1; lvl < 3; ++lvl) {
      histogram_pass(lvl, prefix, mask);
      find_bin(sh, kBins[lvl], need);
      need -= sh.sel_above;
      prefix |= sh.sel_bin << kShift[lvl];
      mask |= (uint32_t)(kBins[lvl] - 1) << kShift[lvl];
      __syncthreads();                      // sel_* read by all before the next level
    }
  }
  // selected: key > K, and the first `need` keys equal to K in column order
  const uint32_t K = take_all ? 0u : prefix;
  const uint32_t need_eq = take_all ? 0u : need;
  const uint32_t n_sel = take_all ? n_cand : (uint32_t)p.topk;

  // ---- ordered write: 4 consecutive columns per thread per tile ------------
  constexpr int kTile = 4 * kTopkThreads;
  uint64_t carry = 0;                         // (equal << 32) | greater, before the tile
  for (int c0 = 0; c0 < n; c0 += kTile) {
    const int c = c0 + 4 * t;
    uint32_t kk[4];
    uint32_t g = 0, q = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      kk[u] = c + u < n ? src.key(c + u) : kKeyNegInf;
      // every candidate when all are taken (a NaN with all bits set has key 0)
      const bool valid = kk[u] != kKeyNegInf;
      g += (valid && (take_all || kk[u] > K)) ? 1u : 0u;
      q += (valid && !take_all && kk[u] == K) ? 1u : 0u;
    }
    uint64_t tile_total;
    const uint64_t before =
        carry + block_exclusive_scan<uint64_t>(((uint64_t)q << 32) | g, sh.wave_sums64, &tile_total);
    uint32_t gb = (uint32_t)before, qb = (uint32_t)(before >> 32);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool valid = kk[u] != kKeyNegInf;
      if (valid && (take_all || kk[u] > K)) {
        const uint32_t pos = gb + min(qb, need_eq);
        if (pos < (uint32_t)p.topk) out[pos] = s + c + u;
        ++gb;
      } else if (valid && kk[u] == K) {
        if (qb < need_eq) {
          const uint32_t pos = gb + qb;
          if (pos < (uint32_t)p.topk) out[pos] = s + c + u;
        }
        ++qb;
      }
    }
    carry += tile_total;
  }
  for (int pos = (int)n_sel + t; pos < p.topk; pos += kTopkThreads) out[pos] = -1;
}

template <int IN>
__global__ __launch_bounds__(kTopkThreads) void topk_stream_kernel(TopkParams p) {
  __shared__ TopkShared sh;
  __shared__ TopkLists ls;
  topk_stream_row<IN>(p, blockIdx.x, sh, ls);
}

// One radix level over a 256-bin histogram h (bin 255 holds the largest
// keys): the bin holding the need-th largest key, the count in higher bins
// and the bin's own count.  Every wave reads the histogram and reaches the
// same answer, so no second barrier is needed.  1 <= need <= the total.
struct BinPick {
  uint32_t bin, above, count;
};
__device__ __forceinline__ BinPick pick_bin256(const uint32_t* h, uint32_t need) {
  const int lane = threadIdx.x & (kWaveLanes - 1);
  typedef uint32_t v4u __attribute__((ext_vector_type(4)));
  uint32_t local;
  {
    const v4u v = *reinterpret_cast<const v4u*>(h + 252 - 4 * lane);   // bins 252-4l .. 255-4l
    local = v[0] + v[1] + v[2] + v[3];
  }
  const uint32_t incl = wave_scan_u32(local, 0u, OpAdd{});
  // the lane whose four bins reach need; its bins are read again (one address
  // for the whole wave) and searched on the scalar unit
  const uint64_t hit = __ballot(incl - local < need && incl >= need);
  const int src = hit ? __builtin_ctzll(hit) : 0;
  uint32_t run = (uint32_t)__builtin_amdgcn_readlane((int)(incl - local), src);
  const v4u w = *reinterpret_cast<const v4u*>(h + 252 - 4 * src);
  uint32_t bin = 255 - 4 * src, cnt = 0;
#pragma unroll
  for (int j = 3; j >= 0; --j, --bin) {      // bins 255-4src down to 252-4src
    cnt = (uint32_t)__builtin_amdgcn_readfirstlane((int)w[j]);
    if (run + cnt >= need) break;
    run += cnt;
  }
  return {bin, run, cnt};
}

// ---- the prefilter of the register kernels ----------------------------------
// A threshold T is taken from a sample of the row's keys (kSamples per
// thread, from tiles spread over the row), at the sample's r-th largest key
// with r set so that the row holds at least topk keys >= T by a margin of
// three standard deviations of the sampling and well under the list's
// capacity.  A wave counts its keys >= T (and its candidates), reserves that
// many slots of an LDS list with one atomic and appends the keys with their
// columns (ballot offsets); the radix levels then run over that list only,
// over the bits in which T and the row's largest key differ (8 bits a level,
// each wave scanning the histogram itself), and the selection is marked in
// LDS bitmaps over the columns from the list.  A row with at most topk
// candidates takes them all.  If the row holds fewer than topk keys >= T, or
// the list overflows, a full selection runs instead: the result is the same,
// only slower.

// The prefilter's per-wave figures.
struct PrefilterLds {
  uint32_t smp[3][kTopkWaves];   // sample minimum, maximum, in-range | valid << 16
  uint32_t list[2][kTopkWaves];  // candidates (counted when needed); largest bits (biased)
  uint32_t count;                // list slots reserved
};

// The threshold T: the lower edge of the sample's bin that holds its rank-r
// key; 0 when the sample holds no candidate.  smp[q] is the key of the
// thread's sampled column scol[q] (kKeyNegInf past the range).
// sh.hist[0, 1024) must be zero; every thread calls it.
template <int kSamples, int kCap>
__device__ __forceinline__ uint32_t prefilter_threshold(const uint32_t (&smp)[kSamples],
                                                        const int (&scol)[kSamples], int n,
                                                        int topk, TopkShared& sh,
                                                        PrefilterLds& pf) {
  const int t = threadIdx.x, lane = t & (kWaveLanes - 1), wave = t >> 6;
  uint32_t vmin = ~0u, vmax = 0, n_in = 0, n_val = 0;
#pragma unroll
  for (int q = 0; q < kSamples; ++q) {
    const uint32_t v = smp[q];
    const bool valid = v != kKeyNegInf;       // columns past the range hold -inf keys
    vmin = valid ? min(vmin, v) : vmin;
    vmax = valid ? max(vmax, v) : vmax;
    n_in += __popcll(__ballot(scol[q] < n));
    n_val += __popcll(__ballot(valid));
  }
  vmin = wave_min_u32(vmin);
  vmax = wave_max_u32(vmax);
  if (lane == 0) {
    pf.smp[0][wave] = vmin;
    pf.smp[1][wave] = vmax;
    pf.smp[2][wave] = n_in | n_val << 16;
  }
  __syncthreads();
  const bool wl = lane < kTopkWaves;
  const uint32_t mn = wave_min_u32(wl ? pf.smp[0][lane] : ~0u);
  const uint32_t mx = wave_max_u32(wl ? pf.smp[1][lane] : 0u);
  const uint32_t packed = wave_sum_u32(wl ? pf.smp[2][lane] : 0u);
  const uint32_t s_in = packed & 0xffffu, s_val = packed >> 16;
  if (s_val == 0) return 0u;
  // A sample key stands for rho row columns; with r sample keys >= T the
  // row's count of keys >= T is about r * rho, with a standard deviation of
  // about rho * sqrt(r).  r solves r * rho - 3 rho sqrt(r) = topk; the
  // refinement stops once at most r_hi sample keys are >= T.
  const float rho = (float)n / (float)s_in;
  const float x = 1.5f + sqrtf(2.25f + (float)topk / rho);
  uint32_t need = min((uint32_t)ceilf(x * x), s_val);
  const uint32_t r_hi = max(need, (uint32_t)(0.7f * (float)kCap / rho));
  uint32_t pre = 0, got = s_val, acc = 0;
  int pos = 32 - __clz(mx - mn);              // offset bits below the common prefix
  for (int lvl = 0; pos > 0 && got > r_hi; ++lvl) {
    const int shf = max(pos - 8, 0);
    uint32_t* h = sh.hist + 256 * lvl;
    const uint32_t fixed = pos >= 32 ? 0u : ~0u << pos;
#pragma unroll
    for (int q = 0; q < kSamples; ++q) {
      const uint32_t off = smp[q] - mn;
      if (smp[q] != kKeyNegInf && ((off ^ pre) & fixed) == 0)
        atomicAdd(&h[(off >> shf) & 255u], 1u);
    }
    __syncthreads();
    const BinPick b = pick_bin256(h, need);
    need -= b.above;
    acc += b.above;
    got = acc + b.count;                      // sample keys >= the bin's lower edge
    pre |= b.bin << shf;
    pos = shf;
  }
  return mn + pre;
}

// Appends the keys >= T of kT register-held tiles (tiles tile0 ..
// tile0 + kT - 1 of the row, as fp32 bit patterns with -inf past the range)
// to the list with their columns, and folds their largest bits into lmax.  The compares run on the bit patterns: for
// T at or above +0 (kPos), key >= T exactly when the bits as a signed integer
// reach T's; for T below -0, exactly when the bits as an unsigned integer are
// at most T's (every non-negative value, and the negative ones nearer zero).
// Without t_ok (T not above -inf) nothing is listed.
template <bool kPos, int kT, int kCap>
__device__ __forceinline__ void count_and_list(const uint32_t (&k)[kT][4], int tile0, uint32_t T,
                                               bool t_ok, int32_t& lmax, PrefilterLds& pf,
                                               uint2* list_kc) {
  constexpr int kTile = 4 * kTopkThreads;
  const int t = threadIdx.x, lane = t & (kWaveLanes - 1);
  const uint32_t tb = kPos ? T ^ 0x80000000u : ~T;
  auto passes = [](uint32_t bits, uint32_t thr) {
    return kPos ? (int32_t)bits >= (int32_t)thr : bits <= thr;
  };
  uint32_t wcnt = 0;
#pragma unroll
  for (int m = 0; m < kT; ++m)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      lmax = max(lmax, (int32_t)k[m][u]);
      wcnt += __popcll(__ballot(passes(k[m][u], tb)));
    }
  // the count is formed here, not where it is used (its masks would stay
  // live through the writes)
  asm volatile("" : "+s"(wcnt));
  uint32_t base = 0;
  if (t_ok && lane == 0) base = atomicAdd(&pf.count, wcnt);
  base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
  if (t_ok && base + wcnt <= (uint32_t)kCap) {
    // The compares are made again here: kept from the counting pass, their
    // masks (two scalar registers per key) would not fit.
    uint32_t tb2 = tb;
    asm volatile("" : "+s"(tb2));
    // the columns are formed again here too (kept from the range checks of
    // the loads, one per key would stay live)
    uint32_t col4 = 4 * t + tile0 * kTile;
    asm volatile("" : "+v"(col4));
    uint32_t run = base;
#pragma unroll
    for (int m = 0; m < kT; ++m)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool pass = passes(k[m][u], tb2);
        const uint64_t b = __ballot(pass);
        if (pass) {
          const uint32_t off =
              run + __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32),
                                              __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
          // a copy made here: paired with its column for the 8-byte store,
          // the key itself would take a register pair for its whole life
          uint32_t kv = k[m][u];
          asm volatile("" : "+v"(kv));
          list_kc[off] = make_uint2(kv, col4 + (uint32_t)(m * kTile + u));
        }
        run += __popcll(b);
      }
  }
}

// After every wave's count_and_list: publishes the wave's largest bits,
// waits for the block, and returns the list's length; U receives a key at or
// above every listed key (the largest non-negative value's, or -0's when
// every value is negative).
__device__ __forceinline__ uint32_t list_totals(int32_t lmax, PrefilterLds& pf, uint32_t& U) {
  const int lane = threadIdx.x & (kWaveLanes - 1), wave = threadIdx.x >> 6;
  const uint32_t wmax = wave_max_u32((uint32_t)lmax ^ 0x80000000u);   // signed order
  if (lane == 0) pf.list[1][wave] = wmax;
  __syncthreads();
  const bool wl = lane < kTopkWaves;
  const int32_t max_bits = (int32_t)(wave_max_u32(wl ? pf.list[1][lane] : 0u) ^ 0x80000000u);
  U = max_bits >= 0 ? (uint32_t)max_bits | 0x80000000u : 0x7FFFFFFFu;
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)pf.count);
}

// The selection from a complete list of `total` (>= topk) keys >= T, all at
// most U: radix levels over the bits where T and U differ (histograms in
// sh.hist[1024, 2048), zero), then the marks of the listed columns in gmap
// (key > K) and qmap (key == K).  Every thread calls it.
__device__ __forceinline__ void list_select_mark(uint32_t total, uint32_t T, uint32_t U, int topk,
                                                 TopkShared& sh, const uint2* list_kc,
                                                 uint32_t* gmap, uint32_t* qmap, uint32_t& K,
                                                 uint32_t& need_eq) {
  const int t = threadIdx.x;
  uint32_t need = (uint32_t)topk;
  int pos = 32 - __clz(U ^ T);
  uint32_t prefix = pos >= 32 ? 0u : U & (~0u << pos);
  bool whole = false;
  for (int lvl = 0; pos > 0; ++lvl) {
    const int shf = max(pos - 8, 0);
    uint32_t* h = sh.hist + 1024 + 256 * lvl;
    const uint32_t fixed = pos >= 32 ? 0u : ~0u << pos;
    for (int i = t; i < (int)total; i += kTopkThreads) {
      const uint32_t key = order_key(list_kc[i].x);
      if (((key ^ prefix) & fixed) == 0) atomicAdd(&h[(key >> shf) & 255u], 1u);
    }
    __syncthreads();
    const BinPick b = pick_bin256(h, need);
    need -= b.above;
    prefix |= b.bin << shf;
    pos = shf;
    if (pos > 0 && b.count == need && prefix != 0) {   // the whole bin is taken
      whole = true;
      break;
    }
  }
  K = whole ? prefix - 1u : prefix;
  need_eq = whole ? 0u : need;
  for (int i = t; i < (int)total; i += kTopkThreads) {
    const uint2 e = list_kc[i];
    const uint32_t key = order_key(e.x);
    const int c = (int)e.y;
    if (key > K) atomicOr(&gmap[c >> 5], 1u << (c & 31));
    else if (key == K) atomicOr(&qmap[c >> 5], 1u << (c & 31));
  }
}

// ---- ordered write ---------------------------------------------------------
// The block walks the bitmaps gmap (key > K) and qmap (key == K) one
// 32-column word at a time in column order: a scan of the words' counts
// gives each word's first output slot and how many of its == K columns are
// still taken (the first need_eq in column order); each word's columns are
// written in ascending order (column s + the word's bit), then -1 up to topk.
// Every thread calls it, after the bitmaps are complete.
template <int kWords>
__device__ __forceinline__ void ordered_write(const uint32_t* gmap, const uint32_t* qmap,
                                              uint32_t need_eq, int topk, int s, int32_t* out,
                                              TopkShared& sh) {
  const int t = threadIdx.x;
  constexpr int kWpt = (kWords + kTopkThreads - 1) / kTopkThreads;   // per thread
  uint32_t wg[kWpt], wq[kWpt];
  uint32_t cg = 0, cq = 0;
#pragma unroll
  for (int j = 0; j < kWpt; ++j) {
    const int w = t * kWpt + j;
    wg[j] = w < kWords ? gmap[w] : 0u;
    wq[j] = w < kWords ? qmap[w] : 0u;
    cg += __popc(wg[j]);
    cq += __popc(wq[j]);
  }
  uint64_t total;
  const uint64_t before =
      block_exclusive_scan<uint64_t>(((uint64_t)cq << 32) | cg, sh.wave_sums64, &total);
  uint32_t gb = (uint32_t)before, qb = (uint32_t)(before >> 32);
  // columns written: all keys > K, then need_eq of the == K ones (topk, or
  // every candidate when all are taken)
  const uint32_t n_sel =
      min((uint32_t)topk, (uint32_t)total + min(need_eq, (uint32_t)(total >> 32)));
#pragma unroll
  for (int j = 0; j < kWpt; ++j) {
    // the == K columns of this word still taken: the lowest `take` set bits
    // the == K columns placed before this word, and how many of this word's
    // are taken.  Written without a guarded subtraction: as
    // `qb < need_eq ? min(need_eq - qb, nq) : 0`, LLVM evaluated the
    // subtraction unconditionally with its no-wrap flag and then folded
    // min(qb, need_eq) below to qb, a wrong position when qb > need_eq.
    const uint32_t nq = __popc(wq[j]);
    const uint32_t placed = min(qb, need_eq);
    uint32_t take = min(need_eq - placed, nq);
    uint32_t sel_q = 0, rest = wq[j];
    for (; take > 0; --take) {
      const uint32_t low = rest & (0u - rest);
      sel_q |= low;
      rest ^= low;
    }
    uint32_t word = wg[j] | sel_q;
    uint32_t pos = gb + placed;
    const int col0 = s + 32 * (t * kWpt + j);
    while (word) {
      const int b = __builtin_ctz(word);
      word &= word - 1;
      if (pos < (uint32_t)topk) out[pos] = col0 + b;
      ++pos;
    }
    gb += __popc(wg[j]);
    qb += nq;
  }
  for (int pos = (int)n_sel + t; pos < topk; pos += kTopkThreads) out[pos] = -1;
}

// Rows of up to kTopkThreads * R columns (R up to 32): the row is read once,
// into registers (thread t holds columns 4t .. 4t+3 of every 4096-column
// tile, so the loads coalesce), and the selection works from there: the
// prefilter above (rows longer than topk, topk up to half the list), else a
// full selection: the first level histograms every key (11 bits), the keys
// in its bin are gathered into LDS and the finer levels histogram that short
// list; the selection is marked in the bitmaps from the registers.  The
// bitmaps give column order directly (ordered_write).
// Up to 32 keys per thread: at most 64 VGPRs, so two blocks (8 waves per
// SIMD) share a compute unit and one block's loads overlap the other's work.
template <int IN, int R>
__global__ __launch_bounds__(kTopkThreads, 8) void topk_reg_kernel(TopkParams p) {
  static_assert(R % 4 == 0 && R <= 32, "whole 4-column groups; 64 VGPRs");
  constexpr int kTiles = R / 4;
  constexpr int kTile = 4 * kTopkThreads;
  constexpr int kWords = kTiles * kTile / 32;  // 32-column words of the register-held row
  constexpr int kCap = 5120;                   // LDS list: prefilter keys, or one bin's keys
  constexpr int kSamples = R >= 32 ? R / 16 : 1;   // sample keys per thread
  static_assert((kTiles & (kTiles - 1)) == 0 && kTiles % kSamples == 0, "sample tiles");
  __shared__ TopkShared sh;
  __shared__ union {
    uint32_t hist_more[3 * kHistStride];      // copies 1..3 of the first-level histogram
    uint32_t maps[2 * kWords];                // then the column bitmaps (key > K, key == K)
  } u_;
  uint32_t* const hist_more = u_.hist_more;
  uint32_t* const gmap = u_.maps;
  uint32_t* const qmap = u_.maps + kWords;
  __shared__ uint2 list_kc[kCap];             // the prefilter's (bit pattern, column) pairs
  uint32_t* const bin_keys = reinterpret_cast<uint32_t*>(list_kc);   // or the first-level bin's keys
  __shared__ PrefilterLds pf;
  __shared__ uint32_t bin_count;
  const int t = threadIdx.x;
  const int lane = t & (kWaveLanes - 1);
  const int64_t row = blockIdx.x;
  int s = 0, e = p.skv;
  if (p.k_start) {
    s = clampi(p.k_start[row], 0, p.skv);
    e = clampi(p.k_end[row], s, p.skv);
  }
  const int n = e - s;                        // <= kTopkThreads * R (host dispatch)
  constexpr int kIB = IN == kBF16 ? 2 : 4;
  // The buffer ends with the range: loads past it read zeros without going to
  // memory (short ranges read only their columns), and the masks below turn
  // them into -inf.
  const TopkRow<IN> src{make_rsrc(static_cast<const char*>(p.logits) + row * p.stride * kIB,
                                  (uint32_t)(e * kIB)),
                        s, n - 1};
  int32_t* out = p.indices + row * p.out_stride;

  // The row's fp32 bit patterns, -inf past the range (only a tile the range
  // ends in is checked); the prefilter compares them as they are, the other
  // paths turn them into keys first.
  uint32_t k[kTiles][4];
#pragma unroll
  for (int m = 0; m < kTiles; ++m) src.bits4(m * kTile + 4 * t, n, (m + 1) * kTile <= n, k[m]);

  // keys > K are taken, then the first need_eq keys equal to K in column order
  uint32_t K = 0, need_eq = 0;
  bool take_all = n <= p.topk;                // every candidate is taken
  bool fast = false;                          // the prefilter marked the selection

  if (!take_all && p.topk <= kCap / 2) {
    for (int b = t; b < 2048; b += kTopkThreads) sh.hist[b] = 0;
    for (int w = t; w < 2 * kWords; w += kTopkThreads) u_.maps[w] = 0;
    if (t == 0) pf.count = 0;
    // the sample, from the registers: thread t's first column of tile
    // (t + q kTiles / kSamples) mod kTiles
    uint32_t smp[kSamples];
    int scol[kSamples];
#pragma unroll
    for (int q = 0; q < kSamples; ++q) {
      const int tq = (t + q * (kTiles / kSamples)) & (kTiles - 1);
      uint32_t v = k[0][0];
#pragma unroll
      for (int m = 1; m < kTiles; ++m) v = tq == m ? k[m][0] : v;
      smp[q] = order_key(v);
      scol[q] = tq * kTile + 4 * t;
    }
    const uint32_t T = prefilter_threshold<kSamples, kCap>(smp, scol, n, p.topk, sh, pf);
    const bool t_ok = T > kKeyNegInf;
    int32_t lmax = INT32_MIN;
    if (T >= 0x80000000u) count_and_list<true, kTiles, kCap>(k, 0, T, t_ok, lmax, pf, list_kc);
    else count_and_list<false, kTiles, kCap>(k, 0, T, t_ok, lmax, pf, list_kc);
    uint32_t U;
    const uint32_t total = list_totals(lmax, pf, U);
    if (total < (uint32_t)p.topk) {           // too few keys >= T: count the candidates
      uint32_t cand = 0;
#pragma unroll
      for (int m = 0; m < kTiles; ++m)
#pragma unroll
        for (int u = 0; u < 4; ++u) cand += __popcll(__ballot(k[m][u] != kBitsNegInf));
      if (lane == 0) pf.list[0][t >> 6] = cand;
      __syncthreads();
      const uint32_t n_cand = wave_sum_u32(lane < kTopkWaves ? pf.list[0][lane] : 0u);
      take_all = n_cand <= (uint32_t)p.topk;
    }
    fast = t_ok && total >= (uint32_t)p.topk && total <= (uint32_t)kCap;
    if (fast) list_select_mark(total, T, U, p.topk, sh, list_kc, gmap, qmap, K, need_eq);
  }

  if (!fast) {
    // keys for the full selection and the take-all marks
#pragma unroll
    for (int m = 0; m < kTiles; ++m)
#pragma unroll
      for (int u = 0; u < 4; ++u) k[m][u] = order_key(k[m][u]);
    if (!take_all) {
      // ---- first level: every key, no branch; -inf counts into a spare slot --
      // Each quarter of a wave counts into its own copy of the histogram (most
      // keys fall in a few bins), folded before the search.
      const int copy = lane >> 4;
      for (int b = t; b < kHistStride; b += kTopkThreads) sh.hist[b] = 0;
      for (int b = t; b < 3 * kHistStride; b += kTopkThreads) hist_more[b] = 0;
      if (t == 0) bin_count = 0;
      __syncthreads();
      {
        uint32_t* h = copy > 0 ? hist_more + (copy - 1) * kHistStride : sh.hist;
#pragma unroll
        for (int m = 0; m < kTiles; ++m)
#pragma unroll
          for (int u = 0; u < 4; ++u)
            atomicAdd(&h[k[m][u] != kKeyNegInf ? (k[m][u] >> 21) : 2048u], 1u);
      }
      __syncthreads();
      uint32_t n_cand;
      {
        uint32_t local = 0;
        for (int b = t; b < 2048; b += kTopkThreads) {
          const uint32_t c = sh.hist[b] + hist_more[b] + hist_more[kHistStride + b] +
                             hist_more[2 * kHistStride + b];
          local += c;
          sh.hist[b] = c;                     // copy 0 becomes the folded histogram
        }
        block_exclusive_scan<uint32_t>(local, sh.wave_sums32, &n_cand);
      }
      take_all = n_cand <= (uint32_t)p.topk;
      if (!take_all) {
        uint32_t need = (uint32_t)p.topk;
        find_bin(sh, 2048, need);
        const uint32_t in_bin = sh.hist[sh.sel_bin];
        need -= sh.sel_above;
        uint32_t prefix = sh.sel_bin << 21, mask = 2047u << 21;
        __syncthreads();
        bool whole_bin = in_bin == need && prefix != 0;
        if (!whole_bin) {
          const bool listed = in_bin <= (uint32_t)kCap;
          if (listed) {                       // gather the bin's keys
#pragma unroll
            for (int m = 0; m < kTiles; ++m)
#pragma unroll
              for (int u = 0; u < 4; ++u)
                if (k[m][u] != kKeyNegInf && (k[m][u] & mask) == prefix) {
                  const uint32_t slot = atomicAdd(&bin_count, 1u);
                  if (slot < (uint32_t)kCap) bin_keys[slot] = k[m][u];
                }
            __syncthreads();
          }
          constexpr int kShift[3] = {21, 10, 0};
          constexpr int kBins[3] = {2048, 2048, 1024};
#pragma unroll
          for (int lvl = 1; lvl < 3; ++lvl) {
            for (int b = t; b < kBins[lvl]; b += kTopkThreads) sh.hist[b] = 0;
            __syncthreads();
            if (listed) {
              for (int i = t; i < (int)in_bin; i += kTopkThreads) {
                const uint32_t key = bin_keys[i];
                if ((key & mask) == prefix)
                  atomicAdd(&sh.hist[(key >> kShift[lvl]) & (kBins[lvl] - 1)], 1u);
              }
            } else {
#pragma unroll
              for (int m = 0; m < kTiles; ++m)
#pragma unroll
                for (int u = 0; u < 4; ++u)
                  if (k[m][u] != kKeyNegInf && (k[m][u] & mask) == prefix)
                    atomicAdd(&sh.hist[(k[m][u] >> kShift[lvl]) & (kBins[lvl] - 1)], 1u);
            }
            __syncthreads();
            find_bin(sh, kBins[lvl], need);
            need -= sh.sel_above;
            const uint32_t c = sh.hist[sh.sel_bin];
            prefix |= sh.sel_bin << kShift[lvl];
            mask |= (uint32_t)(kBins[lvl] - 1) << kShift[lvl];
            __syncthreads();
            if (c == need && lvl == 1 && prefix != 0) {   // the whole finer bin is taken
              whole_bin = true;
              break;
            }
          }
        }
        K = whole_bin ? prefix - 1u : prefix;
        need_eq = whole_bin ? 0u : need;
      }
    }
    // ---- the selection's bitmaps from the registers -------------------------
    for (int w = t; w < 2 * kWords; w += kTopkThreads) u_.maps[w] = 0;
    __syncthreads();
#pragma unroll
    for (int m = 0; m < kTiles; ++m) {
      uint32_t ng = 0, nq = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        // every candidate when all are taken (a NaN with all bits set has key 0)
        const bool valid = k[m][u] != kKeyNegInf;
        ng |= (valid && (take_all || k[m][u] > K)) ? 1u << u : 0u;
        nq |= (valid && !take_all && k[m][u] == K) ? 1u << u : 0u;
      }
      const int c = m * kTile + 4 * t;        // the 4 columns' word and bit
      if (ng) atomicOr(&gmap[c >> 5], ng << (c & 31));
      if (nq) atomicOr(&qmap[c >> 5], nq << (c & 31));
    }
  }
  __syncthreads();

  ordered_write<kWords>(gmap, qmap, need_eq, p.topk, s, out, sh);
}

// Rows of up to kParts * 32768 columns (kParts = 2: 32769 .. 65536; 4: up to
// 131072): the register kernel's prefilter with the row loaded in kParts
// parts of 32 keys per thread (each counted and listed in turn), so the block
// stays within 64 VGPRs and about 73 KB of LDS and two blocks share a compute
// unit; the sample (4 keys per thread and 32768 columns) is loaded apart,
// before the row.  A row the prefilter does not settle (at most topk
// candidates, topk above half the list, too few keys >= T, a full list) is
// read again by the streaming selection.
template <int IN, int kParts>
__global__ __launch_bounds__(kTopkThreads, 8) void topk_parts_kernel(TopkParams p) {
  static_assert(kParts == 2 || kParts == 4, "two or four parts");
  constexpr int kHalf = 8;                     // tiles per part
  constexpr int kTiles = kParts * kHalf;
  constexpr int kTile = 4 * kTopkThreads;
  constexpr int kWords = kTiles * kTile / 32;
  constexpr int kCap = kParts == 2 ? 6144 : 4096;
  constexpr int kSamples = 2 * kParts;
  __shared__ TopkShared sh;
  __shared__ union {
    struct {
      uint32_t maps[2 * kWords];              // the column bitmaps (key > K, key == K)
      uint2 list_kc[kCap];                    // the prefilter's (bit pattern, column) pairs
    } f;
    TopkLists ls;                             // the streaming selection's lists
  } u_;
  __shared__ PrefilterLds pf;
  const int t = threadIdx.x;
  const int64_t row = blockIdx.x;
  int s = 0, e = p.skv;
  if (p.k_start) {
    s = clampi(p.k_start[row], 0, p.skv);
    e = clampi(p.k_end[row], s, p.skv);
  }
  const int n = e - s;
  if (n <= p.topk || p.topk > kCap / 2) {
    topk_stream_row<IN>(p, row, sh, u_.ls);
    return;
  }
  constexpr int kIB = IN == kBF16 ? 2 : 4;
  // the buffer ends with the range (loads past it read zeros, masked to -inf)
  const TopkRow<IN> src{make_rsrc(static_cast<const char*>(p.logits) + row * p.stride * kIB,
                                  (uint32_t)(e * kIB)),
                        s, n - 1};
  int32_t* out = p.indices + row * p.out_stride;

  // the sample, loaded: thread t's first column of tile (wave + q kTiles /
  // kSamples) mod kTiles (one tile per wave and load, so a wave's loads fall
  // on adjacent lines)
  uint32_t smp[kSamples];
  int scol[kSamples];
  const int wave = t >> 6;
#pragma unroll
  for (int q = 0; q < kSamples; ++q) {
    scol[q] = ((wave + q * (kTiles / kSamples)) & (kTiles - 1)) * kTile + 4 * t;
    smp[q] = scol[q] < n ? src.key(scol[q]) : kKeyNegInf;
  }
  for (int b = t; b < 2048; b += kTopkThreads) sh.hist[b] = 0;
  for (int w = t; w < 2 * kWords; w += kTopkThreads) u_.f.maps[w] = 0;
  if (t == 0) pf.count = 0;
  const uint32_t T = prefilter_threshold<kSamples, kCap>(smp, scol, n, p.topk, sh, pf);
  const bool t_ok = T > kKeyNegInf;
  int32_t lmax = INT32_MIN;
#pragma nounroll
  for (int h = 0; h < kParts; ++h) {
    uint32_t k[kHalf][4];
#pragma unroll
    for (int m = 0; m < kHalf; ++m) {
      const int tile = h * kHalf + m;
      src.bits4(tile * kTile + 4 * t, n, (tile + 1) * kTile <= n, k[m]);
    }
    if (T >= 0x80000000u) count_and_list<true, kHalf, kCap>(k, h * kHalf, T, t_ok, lmax, pf, u_.f.list_kc);
    else count_and_list<false, kHalf, kCap>(k, h * kHalf, T, t_ok, lmax, pf, u_.f.list_kc);
  }
  uint32_t U;
  const uint32_t total = list_totals(lmax, pf, U);
  if (!t_ok || total < (uint32_t)p.topk || total > (uint32_t)kCap) {
    __syncthreads();                          // the lists reuse the prefilter's LDS
    topk_stream_row<IN>(p, row, sh, u_.ls);
    return;
  }
  uint32_t K, need_eq;
  list_select_mark(total, T, U, p.topk, sh, u_.f.list_kc, u_.f.maps, u_.f.maps + kWords, K,
                   need_eq);
  __syncthreads();
  ordered_write<kWords>(u_.f.maps, u_.f.maps + kWords, need_eq, p.topk, s, out, sh);
}

template <int IN>
static hipError_t launch_topk_in(const TopkParams& p, hipStream_t s) {
  const dim3 grid((unsigned)p.sq), block(kTopkThreads);
  if (p.skv <= 8 * kTopkThreads) {
    hipLaunchKernelGGL((topk_reg_kernel<IN, 8>), grid, block, 0, s, p);
  } else if (p.skv <= 16 * kTopkThreads) {
    hipLaunchKernelGGL((topk_reg_kernel<IN, 16>), grid, block, 0, s, p);
  } else if (p.skv <= 32 * kTopkThreads) {
    hipLaunchKernelGGL((topk_reg_kernel<IN, 32>), grid, block, 0, s, p);
  } else if (p.skv <= 64 * kTopkThreads) {
    hipLaunchKernelGGL((topk_parts_kernel<IN, 2>), grid, block, 0, s, p);
  } else if (p.skv <= 128 * kTopkThreads) {
    hipLaunchKernelGGL((topk_parts_kernel<IN, 4>), grid, block, 0, s, p);
  } else {
    hipLaunchKernelGGL((topk_stream_kernel<IN>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_topk(int in_type, const TopkParams& p, hipStream_t s) {
  if (p.sq == 0) return hipSuccess;
  return in_type == kBF16 ? launch_topk_in<kBF16>(p, s) : launch_topk_in<kF32>(p, s);
}

}  // namespace mqa
