// Even split of a work list over workers, computed on the device by one block
// (the metadata calls of the paged and the dense paths).
//
// Item b (a paged sequence, a dense 4-row group) contributes units(b) >= 0
// work units (b, 0) .. (b, units(b) - 1); the W units in item-major order are
// cut into num_splits contiguous pieces, piece c = units
// [floor(c W / num_splits), floor((c + 1) W / num_splits)), and sched[c] =
// (b, k) of the first unit of piece c, or (n_items, 0) when that unit is W.
#pragma once

#include "common.hpp"

namespace mqa {

constexpr int kMetaThreads = 1024;
constexpr int kMetaMaxItems = 8192;

// Call from every thread of a single block of kMetaThreads threads;
// n_items <= kMetaMaxItems.
template <class Units>
__device__ __forceinline__ void split_units(int n_items, int num_splits, int32_t* sched,
                                            Units&& units) {
  __shared__ int32_t prefix[kMetaMaxItems + 1];
  __shared__ int32_t part[kMetaThreads];
  const int t = threadIdx.x;
  constexpr int kPer = kMetaMaxItems / kMetaThreads;   // items per thread
  int local[kPer];
  int sum = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int b = t * kPer + k;
    const int nb = b < n_items ? units(b) : 0;
    local[k] = nb;
    sum += nb;
  }
  part[t] = sum;
  __syncthreads();
  for (int step = 1; step < kMetaThreads; step <<= 1) {   // inclusive scan
    const int v = t >= step ? part[t - step] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int run = part[t] - sum;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int b = t * kPer + k;
    if (b <= n_items) prefix[b] = run;
    run += local[k];
  }
  if (t == kMetaThreads - 1 && n_items == kMetaMaxItems) prefix[n_items] = part[t];
  __syncthreads();
  const int64_t total = prefix[n_items];
  for (int c = t; c <= num_splits; c += kMetaThreads) {
    const int64_t u = (int64_t)c * total / num_splits;
    int sb = n_items, sk = 0;
    if (u < total) {
      int lo = 0, hi = n_items;            // largest b with prefix[b] <= u
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (prefix[mid] <= u) lo = mid; else hi = mid;
      }
      sb = lo;
      sk = (int)(u - prefix[lo]);
    }
    sched[2 * c] = sb;
    sched[2 * c + 1] = sk;
  }
}

}  // namespace mqa
