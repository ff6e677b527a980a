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

// Codes -> fp32 with the gfx950 conversion instructions (exact; e4m3 is the
// OCP e4m3fn format, e2m1 elements low nibble first):
// four e4m3 codes of a word, or the four e2m1 codes of its low 16 bits.
template <int FMT>
__device__ __forceinline__ void decode4(uint32_t word, float (&v)[4]) {
  typedef float v2f __attribute__((ext_vector_type(2)));
  v2f a, b;
  if constexpr (FMT == kMXFP4) {
    a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 0);
    b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 1);
  } else {
    a = __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
    b = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);
  }
  v[0] = a[0];
  v[1] = a[1];
  v[2] = b[0];
  v[3] = b[1];
}

// Thread t of a row handles elements 4t .. 4t+3 (one dword of fp8 codes, two
// bytes of fp4 codes per head); 8 consecutive threads cover one 32-element
// scale block.  kRowsPerBlock rows per block of 256 threads.
template <int D>
struct QsumShape {
  static constexpr int kThreadsPerRow = D / 4;
  static constexpr int kRowsPerBlock = 256 / kThreadsPerRow;
};

template <int FMT, int H, int D, bool WBF16>
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
  const uint8_t* qrow = p.q + i * H * kRowBytes;
#pragma unroll
  for (int h = 0; h < H; ++h) {
    if constexpr (FMT == kMXFP4) {
      code[h] = *reinterpret_cast<const uint16_t*>(qrow + h * kRowBytes + (k0 >> 1));
    } else {
      code[h] = *reinterpret_cast<const uint32_t*>(qrow + h * kRowBytes + k0);
    }
    if constexpr (FmtInfo<FMT>::kMX) sf[h] = p.q_sf[(i * H + h) * kNKB + (k0 >> 5)];
    if constexpr (WBF16) {
      wt[h] = bf16_value(static_cast<const uint16_t*>(p.w)[i * H + h]);
    } else {
      wt[h] = static_cast<const float*>(p.w)[i * H + h];
    }
  }
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int h = 0; h < H; ++h) {
    float wh = 0.5f * wt[h];
    if constexpr (FmtInfo<FMT>::kMX) wh = ldexpf(wh, (int)sf[h] - 127);   // the block scale
    float v[4];
    decode4<FMT>(code[h], v);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(wh, v[e], acc[e]);
  }

  // Four pieces: each takes the block's residual at the largest e8m0 scale
  // that keeps every element within e4m3's range (|x| 2^-sc <= 448), rounded
  // to e4m3 (nearest, ties to even: v_cvt_pk_fp8_f32).
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
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(r[0], -sc), ldexpf(r[1], -sc), 0, false);
    const uint32_t word =
        (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(r[2], -sc), ldexpf(r[3], -sc), lo, true);
    float back[4];
    decode4<kFP8>(word, back);
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] -= ldexpf(back[e], sc);
    const int64_t pr = i * 4 + piece;
    *reinterpret_cast<uint32_t*>(p.ql + pr * D + k0) = word;
    if ((t & 7) == 0) p.ql_sf[pr * kNKB + (k0 >> 5)] = (uint8_t)(sc + 127);
  }
}

template <int FMT, int D>
static hipError_t launch_qsum_inst(const QsumParams& p, hipStream_t s) {
  using S = QsumShape<D>;
  const int blocks = (p.sq + S::kRowsPerBlock - 1) / S::kRowsPerBlock;
  if (p.w_bf16) {
    hipLaunchKernelGGL((qsum_kernel<FMT, 64, D, true>), dim3(blocks), dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL((qsum_kernel<FMT, 64, D, false>), dim3(blocks), dim3(256), 0, s, p);
  }
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
