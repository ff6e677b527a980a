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
// keys (sign-magnitude to two's-complement order), and a three-level radix
// select (11 + 11 + 10 bits, one LDS histogram per level, each level a pass
// over the row) finds the k-th largest key K and how many equal keys to keep.
// A last pass writes the selected columns in column order with a block-wide
// prefix count of (keys > K, keys == K).
#include "common.hpp"
#include "launch.hpp"

namespace mqa {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWaveLanes;
constexpr uint32_t kKeyNegInf = 0x007FFFFFu;       // key of -inf: not a candidate

// Order-preserving key of an fp32 bit pattern: larger float, larger key.
__device__ __forceinline__ uint32_t order_key(uint32_t bits) {
  return (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
}

template <int IN>
struct TopkRow {
  Rsrc r;
  int s;                                  // first column of the range (element offset)
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
};

// Exclusive prefix sum over the block (thread order) of a per-thread value;
// *total receives the block total.  Every thread must call it.
template <class T>
__device__ __forceinline__ T block_exclusive_scan(T v, T* wave_sums, T* total) {
  const int lane = threadIdx.x & (kWaveLanes - 1);
  const int wave = threadIdx.x >> 6;
  T x = v;
#pragma unroll
  for (int o = 1; o < kWaveLanes; o <<= 1) {
    const T y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == kWaveLanes - 1) wave_sums[wave] = x;
  __syncthreads();
  if (wave == 0) {
    T w = lane < kTopkWaves ? wave_sums[lane] : T(0);
#pragma unroll
    for (int o = 1; o < kTopkWaves; o <<= 1) {
      const T y = __shfl_up(w, o);
      if (lane >= o) w += y;
    }
    if (lane < kTopkWaves) wave_sums[lane] = w;             // inclusive per wave
  }
  __syncthreads();
  const T before = wave > 0 ? wave_sums[wave - 1] : T(0);
  *total = wave_sums[kTopkWaves - 1];
  __syncthreads();                                          // wave_sums reusable after this
  return before + x - v;
}

struct TopkShared {
  uint32_t hist[2048];
  uint64_t wave_sums64[kTopkWaves];
  uint32_t wave_sums32[kTopkWaves];
  uint32_t sel_bin, sel_above;
};

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

template <int IN>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkParams p) {
  __shared__ TopkShared sh;
  const int t = threadIdx.x;
  const int64_t row = blockIdx.x;
  int s = 0, e = p.skv;
  if (p.k_start) {
    s = clampi(p.k_start[row], 0, p.skv);
    e = clampi(p.k_end[row], s, p.skv);
  }
  const int n = e - s;
  constexpr int kIB = IN == kBF16 ? 2 : 4;
  const TopkRow<IN> src{make_rsrc(static_cast<const char*>(p.logits) + row * p.stride * kIB,
                                  (uint32_t)(p.skv * kIB)),
                        s};
  int32_t* out = p.indices + row * p.out_stride;

  // ---- three radix levels: K = the topk-th largest candidate key ----------
  constexpr int kShift[3] = {21, 10, 0};
  constexpr int kBins[3] = {2048, 2048, 1024};
  uint32_t need = (uint32_t)p.topk;         // keys still to place at or below the prefix
  uint32_t prefix = 0, mask = 0;
  uint32_t n_cand = 0;
  bool take_all = false;
#pragma unroll
  for (int lvl = 0; lvl < 3; ++lvl) {
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
    if (lvl == 0) {
      uint32_t local = 0;
      for (int b = t; b < 2048; b += kTopkThreads) local += sh.hist[b];
      block_exclusive_scan<uint32_t>(local, sh.wave_sums32, &n_cand);
      if (n_cand <= (uint32_t)p.topk) {     // every candidate is selected
        take_all = true;
        break;
      }
    }
    find_bin(sh, kBins[lvl], need);
    need -= sh.sel_above;
    prefix |= sh.sel_bin << kShift[lvl];
    mask |= (uint32_t)(kBins[lvl] - 1) << kShift[lvl];
    __syncthreads();                          // sel_* read by all before the next level
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
      const bool valid = kk[u] != kKeyNegInf;
      g += (valid && kk[u] > K) ? 1u : 0u;
      q += (valid && kk[u] == K) ? 1u : 0u;
    }
    uint64_t tile_total;
    const uint64_t before =
        carry + block_exclusive_scan<uint64_t>(((uint64_t)q << 32) | g, sh.wave_sums64, &tile_total);
    uint32_t gb = (uint32_t)before, qb = (uint32_t)(before >> 32);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool valid = kk[u] != kKeyNegInf;
      if (valid && kk[u] > K) {
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

hipError_t launch_topk(int in_type, const TopkParams& p, hipStream_t s) {
  if (p.sq == 0) return hipSuccess;
  if (in_type == kBF16) {
    hipLaunchKernelGGL(topk_kernel<kBF16>, dim3((unsigned)p.sq), dim3(kTopkThreads), 0, s, p);
  } else {
    hipLaunchKernelGGL(topk_kernel<kF32>, dim3((unsigned)p.sq), dim3(kTopkThreads), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace mqa
