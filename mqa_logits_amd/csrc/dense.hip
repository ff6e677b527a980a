// Dense and compressed weighted MQA logits for gfx950: fp32-logits instances
// split by row chunks, the dispatch over logits type and work split, and the
// compressed layout's row offsets.  The kernels are in dense_kernel.hpp.
#include "dense_kernel.hpp"
#include "schedule.hpp"

namespace mqa {

hipError_t launch_dense_f32(int fmt, int h, int d, int store, const DenseParams& p, hipStream_t s) {
  return dispatch_fmt<kF32, false>(fmt, h, d, store, p, s);
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

// Row offsets of the compressed layout: exclusive prefix sum of the clamped
// row lengths, one block of 1024 threads walking the rows in chunks.
__global__ __launch_bounds__(1024) void compressed_offsets_kernel(const int32_t* __restrict__ ks,
                                                                  const int32_t* __restrict__ ke,
                                                                  int32_t sq, int32_t skv,
                                                                  int64_t* __restrict__ off) {
  __shared__ int64_t part[1024];
  __shared__ int64_t carry_s;
  const int t = threadIdx.x;
  if (t == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base < sq; base += 1024) {
    const int i = base + t;
    int64_t len = 0;
    if (i < sq) {
      const int s = clampi(ks[i], 0, skv);
      const int e = clampi(ke[i], s, skv);
      len = e - s;
    }
    part[t] = len;
    __syncthreads();
    for (int step = 1; step < 1024; step <<= 1) {     // inclusive scan
      const int64_t v = t >= step ? part[t - step] : 0;
      __syncthreads();
      part[t] += v;
      __syncthreads();
    }
    const int64_t carry = carry_s;
    if (i < sq) off[i] = carry + part[t] - len;
    __syncthreads();
    if (t == 1023) carry_s = carry + part[1023];
    __syncthreads();
  }
  if (t == 0) off[sq] = carry_s;
}

hipError_t launch_compressed_offsets(const int32_t* ks, const int32_t* ke, int32_t sq, int32_t skv,
                                     int64_t* off, hipStream_t s) {
  hipLaunchKernelGGL(compressed_offsets_kernel, dim3(1), dim3(1024), 0, s, ks, ke, sq, skv, off);
  return hipGetLastError();
}

}  // namespace mqa
