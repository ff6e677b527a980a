// Dense and compressed weighted MQA logits for gfx950: fp32-logits instances
// split by row chunks, the dispatch over logits type and work split, and the
// compressed layout's row offsets.  The kernels are in dense_kernel.hpp.
#include <type_traits>

#include "dense_kernel.hpp"
#include "schedule.hpp"

namespace mqa {

hipError_t launch_dense_f32(int fmt, int h, int d, int store, const DenseParams& p, hipStream_t s) {
  return dispatch_fmt<kF32, false>(fmt, h, d, store, p.exact != 0, p, s);
}

hipError_t launch_dense(int fmt, int h, int d, int store, int out, const DenseParams& p,
                        hipStream_t s) {
  if (p.sched)
    return out == kBF16 ? launch_dense_sched_bf16(fmt, h, d, store, p, s)
                        : launch_dense_sched_f32(fmt, h, d, store, p, s);
  return out == kBF16 ? launch_dense_bf16(fmt, h, d, store, p, s)
                      : launch_dense_f32(fmt, h, d, store, p, s);
}

// Work schedule of the scheduled kernels: 4-row group g contributes
// max(group_trips, 1) units, counted exactly as dense_group counts them.
__global__ __launch_bounds__(kMetaThreads) void dense_metadata_kernel(
    const int32_t* __restrict__ ks, const int32_t* __restrict__ ke, int32_t sq, int32_t skv,
    int32_t num_splits, int32_t* __restrict__ sched) {
  const int n_groups = (sq + kRowsPerWave - 1) / kRowsPerWave;
  split_units(n_groups, num_splits, sched, [&](int grp) {
    int lo = 0x7fffffff, hi = 0;
    for (int r = 0; r < kRowsPerWave; ++r) {
      const int row = grp * kRowsPerWave + r;
      if (row >= sq) break;
      const int s = clampi(ks[row], 0, skv);
      const int e = clampi(ke[row], s, skv);
      if (e > s) {
        lo = min(lo, s);
        hi = max(hi, e);
      }
    }
    return max(group_trips(lo, hi), 1);
  });
}

hipError_t launch_dense_metadata(const int32_t* ks, const int32_t* ke, int32_t sq, int32_t skv,
                                 int32_t num_splits, int32_t* sched, hipStream_t s) {
  hipLaunchKernelGGL(dense_metadata_kernel, dim3(1), dim3(kMetaThreads), 0, s, ks, ke, sq, skv,
                     num_splits, sched);
  return hipGetLastError();
}

// Inclusive sum over the wave of a 64-bit value with DPP moves (ALU latency,
// no LDS round trips): shifts by 1, 2, 4 and 8 lanes within each row of 16,
// then row 0's and row 1's last lanes broadcast to the rows after them.  Each
// 32-bit half moves on its own and the sum is formed in 64 bits; lanes
// without a source add 0.  Every lane of the wave takes part.
__device__ __forceinline__ int64_t wave_incl_sum_i64(int64_t x) {
  auto step = [&](auto ctrl, auto row_mask) {
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)x, decltype(ctrl)::value,
                                               decltype(row_mask)::value, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)((uint64_t)x >> 32),
                                               decltype(ctrl)::value, decltype(row_mask)::value,
                                               0xf, false);
    x += (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
  };
  step(std::integral_constant<int, 0x111>{}, std::integral_constant<int, 0xf>{});
  step(std::integral_constant<int, 0x112>{}, std::integral_constant<int, 0xf>{});
  step(std::integral_constant<int, 0x114>{}, std::integral_constant<int, 0xf>{});
  step(std::integral_constant<int, 0x118>{}, std::integral_constant<int, 0xf>{});
  step(std::integral_constant<int, 0x142>{}, std::integral_constant<int, 0xa>{});
  step(std::integral_constant<int, 0x143>{}, std::integral_constant<int, 0xc>{});
  return x;
}

// Row offsets of the compressed layout: exclusive prefix sum of the clamped
// row lengths, one block of 1024 threads walking the rows in chunks.
__global__ __launch_bounds__(1024) void compressed_offsets_kernel(const int32_t* __restrict__ ks,
                                                                  const int32_t* __restrict__ ke,
                                                                  int32_t sq, int32_t skv,
                                                                  int64_t* __restrict__ off) {
  // Thread t takes rows 4t .. 4t+3 of each round of 4096; a round is a scan
  // of the threads' sums inside each wave, then of the 16 wave totals (both
  // DPP scans), so it costs three barriers.
  constexpr int kPer = 4;
  constexpr int kWaves = 1024 / kWaveLanes;
  __shared__ int64_t wsum[kWaves];
  const int t = threadIdx.x, lane = t & (kWaveLanes - 1), wave = t / kWaveLanes;
  int64_t carry = 0;
  for (int base = 0; base < sq; base += 1024 * kPer) {
    int64_t len[kPer], tsum = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int i = base + kPer * t + k;
      len[k] = 0;
      if (i < sq) {
        const int s = clampi(ks[i], 0, skv);
        len[k] = clampi(ke[i], s, skv) - s;
      }
      tsum += len[k];
    }
    const int64_t x = wave_incl_sum_i64(tsum);
    if (lane == kWaveLanes - 1) wsum[wave] = x;
    __syncthreads();
    if (wave == 0) {                           // inclusive scan of the wave totals
      const int64_t v = wave_incl_sum_i64(lane < kWaves ? wsum[lane] : 0);
      if (lane < kWaves) wsum[lane] = v;
    }
    __syncthreads();
    int64_t excl = carry + (wave > 0 ? wsum[wave - 1] : 0) + x - tsum;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int i = base + kPer * t + k;
      if (i < sq) off[i] = excl;
      excl += len[k];
    }
    carry += wsum[kWaves - 1];
    __syncthreads();                           // wsum is rewritten by the next round
  }
  if (t == 0) off[sq] = carry;
}

hipError_t launch_compressed_offsets(const int32_t* ks, const int32_t* ke, int32_t sq, int32_t skv,
                                     int64_t* off, hipStream_t s) {
  hipLaunchKernelGGL(compressed_offsets_kernel, dim3(1), dim3(1024), 0, s, ks, ke, sq, skv, off);
  return hipGetLastError();
}

}  // namespace mqa
