// Weighted query sums for the linear half of the ReLU, gfx950.
//
// With H = 64 heads the dense kernels evaluate
//   sum_h w[i,h] ReLU(x_h) = sum_h (w[i,h] / 2) |x_h| + sum_h (w[i,h] / 2) x_h,
// ReLU(x) = (x + |x|) / 2, x_h = <q[i,h,:], kv[j,:]> (the weighted head sum of
// "How to Implement MQA (Multi-Query Attention) Logits Computation with
// DeepGEMM", Core Architecture Components).  The second sum is linear in kv:
// it equals <q'_i, kv[j,:]> with q'_i = sum_h (w[i,h] / 2) q[i,h,:], so the
// matrix core computes it as one extra 16-row tile per 16 tokens instead of a
// max and an fma per head in the vector ALU.  This kernel forms q'_i in fp32
// from the decoded codes (block scales applied) and writes it as four e4m3
// pieces, each with one e8m0 scale per 32 elements, that sum to q'_i to about
// 2^-16 of each block's largest magnitude:
//   ql    [Sq][4][D]     e4m3 codes, piece p of row i at (i * 4 + p) * D
//   ql_sf [Sq][4][D/32]  e8m0 block scales
// -- the layout of an [Sq, 4, D] MXFP8 query tensor, so the dense kernels
// load it like Q.
#include "common.hpp"
#include "launch.hpp"

namespace mqa {

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const int e = (c >> 3) & 15, m = c & 7;
  const float v = e == 0 ? (float)m * 0x1p-9f : ldexpf(1.f + (float)m * 0.125f, e - 7);
  return (c & 0x80) ? -v : v;
}

__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const int e = (c >> 1) & 3, m = c & 1;
  const float v = e == 0 ? 0.5f * (float)m : ldexpf(1.f + 0.5f * (float)m, e - 1);
  return (c & 8) ? -v : v;
}

// Nearest e4m3 code of x, ties to even; |x| <= 448.
__device__ __forceinline__ uint32_t e4m3_rne(float x) {
  const uint32_t s = x < 0.f ? 0x80u : 0u;
  const float a = fabsf(x);
  if (a < 0x1p-6f) {                           // subnormals: multiples of 2^-9
    const uint32_t m = (uint32_t)rintf(a * 0x1p9f);   // 8 is the smallest normal
    return m ? (s | m) : 0u;
  }
  int e;
  const float f = frexpf(a, &e);               // a = f 2^e, f in [0.5, 1)
  uint32_t m = (uint32_t)rintf((2.f * f - 1.f) * 8.f);
  int be = e - 1 + 7;                          // biased exponent of (1 + m/8) 2^(e-1)
  if (m == 8) { m = 0; ++be; }
  return s | ((uint32_t)be << 3) | m;
}

// Thread t of a row handles elements 4t .. 4t+3 (one dword of fp8 codes, two
// bytes of fp4 codes per head); 8 consecutive threads cover one 32-element
// scale block.  kRowsPerBlock rows per block of 256 threads.
template <int D>
struct QsumShape {
  static constexpr int kThreadsPerRow = D / 4;
  static constexpr int kRowsPerBlock = 256 / kThreadsPerRow;
};

template <int FMT, int H, int D>
__global__ __launch_bounds__(256) void qsum_kernel(QsumParams p) {
  using S = QsumShape<D>;
  constexpr int kRowBytes = FMT == kMXFP4 ? D / 2 : D;
  constexpr int kNKB = D / 32;
  const int t = threadIdx.x % S::kThreadsPerRow;
  const int64_t i = (int64_t)blockIdx.x * S::kRowsPerBlock + threadIdx.x / S::kThreadsPerRow;
  if (i >= p.sq) return;                       // whole rows (and scale blocks) leave together
  const int k0 = 4 * t;

  // All H code words, scales and weights of the row are requested before any
  // is used (one memory round trip, not H).
  uint32_t code[H];
  uint32_t sf[FmtInfo<FMT>::kMX ? H : 1];
  float wt[H];
#pragma unroll
  for (int h = 0; h < H; ++h) {
    const int64_t hr = i * H + h;
    if constexpr (FMT == kMXFP4) {
      code[h] = *reinterpret_cast<const uint16_t*>(p.q + hr * kRowBytes + (k0 >> 1));
    } else {
      code[h] = *reinterpret_cast<const uint32_t*>(p.q + hr * kRowBytes + k0);
    }
    if constexpr (FmtInfo<FMT>::kMX) sf[h] = p.q_sf[hr * kNKB + (k0 >> 5)];
    wt[h] = p.w_bf16 ? bf16_value(static_cast<const uint16_t*>(p.w)[hr])
                     : static_cast<const float*>(p.w)[hr];
  }
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int h = 0; h < H; ++h) {
    const float wh = 0.5f * wt[h];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float v = FMT == kMXFP4 ? e2m1_value((code[h] >> (4 * e)) & 15u)
                              : e4m3_value((code[h] >> (8 * e)) & 255u);
      if constexpr (FmtInfo<FMT>::kMX) v = ldexpf(v, (int)sf[h] - 127);
      acc[e] = __builtin_fmaf(wh, v, acc[e]);
    }
  }

  // Four pieces: each takes the block's residual at the largest e8m0 scale
  // that keeps every element within e4m3's range.
  float r[4] = {acc[0], acc[1], acc[2], acc[3]};
#pragma unroll
  for (int piece = 0; piece < 4; ++piece) {
    float m = fmaxf(fmaxf(fabsf(r[0]), fabsf(r[1])), fmaxf(fabsf(r[2]), fabsf(r[3])));
#pragma unroll
    for (int o = 4; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));   // the 8 threads of a block
    int sc = -127;
    if (m > 0.f) {
      int e;
      const float f = frexpf(m, &e);           // m / 2^sc <= 448 = 0.875 * 2^9
      sc = min(max(f <= 0.875f ? e - 9 : e - 8, -127), 127);
    }
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t c = e4m3_rne(ldexpf(r[e], -sc));
      r[e] -= ldexpf(e4m3_value(c), sc);
      word |= c << (8 * e);
    }
    const int64_t pr = i * 4 + piece;
    *reinterpret_cast<uint32_t*>(p.ql + pr * D + k0) = word;
    if ((t & 7) == 0) p.ql_sf[pr * kNKB + (k0 >> 5)] = (uint8_t)(sc + 127);
  }
}

template <int FMT, int D>
static hipError_t launch_qsum_inst(const QsumParams& p, hipStream_t s) {
  using S = QsumShape<D>;
  const int blocks = (p.sq + S::kRowsPerBlock - 1) / S::kRowsPerBlock;
  hipLaunchKernelGGL((qsum_kernel<FMT, 64, D>), dim3(blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_qsum(int fmt, int d, const QsumParams& p, hipStream_t s) {
  if (p.sq == 0) return hipSuccess;
  switch (fmt) {
    case kFP8: return d == 64 ? launch_qsum_inst<kFP8, 64>(p, s) : launch_qsum_inst<kFP8, 128>(p, s);
    case kMXFP8: return d == 64 ? launch_qsum_inst<kMXFP8, 64>(p, s) : launch_qsum_inst<kMXFP8, 128>(p, s);
    default: return d == 64 ? launch_qsum_inst<kMXFP4, 64>(p, s) : launch_qsum_inst<kMXFP4, 128>(p, s);
  }
}

}  // namespace mqa
