// Device-side building blocks shared by the dense, compressed and paged
// weighted-MQA-logits kernels (gfx950 / CDNA4 only).
//
// Tiling used by every kernel (one wave = 64 lanes):
//   * one wave owns 4 query rows and walks KV tokens 16 at a time;
//   * the contraction S[row, head, token] = <q[row, head, :], kv[token, :]>
//     runs on v_mfma_scale_f32_16x16x128_f8f6f4: A = 16 (row, head) pairs x
//     128 elements of D, B = 128 elements x 16 tokens, C = 16 x 16 fp32;
//   * A row r of M tile m is (query row r / 4, head 4m + r % 4).  The
//     accumulator layout puts C rows 4g .. 4g+3 in lanes 16g .. 16g+15, so
//     every accumulator of lane l belongs to query row l / 16 and column
//     l % 16: the weighted ReLU head sum runs entirely inside each lane;
//   * operand lane l carries row/column l % 16 and the pieces of D that its
//     lane group l / 16 holds in the instruction's operand layout
//     (OperandLayout below);
//   * MX block scales ride the MFMA's e8m0 scale operands (127 = 1.0 for the
//     plain FP8 format), so the hardware applies them inside the product.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"

namespace mqa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

enum Fmt : int { kFP8 = 0, kMXFP8 = 1, kMXFP4 = 2 };

constexpr int kWaveLanes = 64;
constexpr int kRowsPerWave = 4;
constexpr int kTileN = 16;
constexpr int kThreads = kWaveLanes * kWavesPerBlock;
constexpr uint32_t kNegInfBits = 0xFF800000u;

template <int FMT>
struct FmtInfo {
  static constexpr bool kMX = FMT != kFP8;
  static constexpr int kCode = FMT == kMXFP4 ? 4 : 0;       // e2m1 : e4m3
};

// Operand layout of v_mfma_scale_f32_16x16x128_f8f6f4 (measured on gfx950):
//   FP4: lane group g (lanes 16g..16g+15) holds elements [32g, 32g+32) of its
//        row in dwords 0..3, and its e8m0 scale byte is block g's;
//   FP8: lane group g holds elements [16g, 16g+16) in dwords 0..3 and
//        [64+16g, 64+16g+16) in dwords 4..7; the hardware applies block
//        (element / 32)'s scale to each, and that scale comes from lane group
//        (element / 32).
// OperandLayout gives, per lane group, the byte offsets inside a row of the
// two 16-byte pieces it loads (-1: the piece is zero).
template <int FMT, int D>
struct OperandLayout {
  static constexpr int kRowBytes = FMT == kMXFP4 ? D / 2 : D;
  static constexpr int kBlocks = D / 32;
  __device__ static constexpr int lo(int g) {
    return FMT == kMXFP4 ? (16 * g < kRowBytes ? 16 * g : -1) : 16 * g;
  }
  __device__ static constexpr int hi(int g) {
    return FMT == kMXFP4 ? -1 : (64 + 16 * g < kRowBytes ? 64 + 16 * g : -1);
  }
  __device__ static constexpr bool scale_ok(int g) { return g < kBlocks; }
};

__device__ __forceinline__ uint4 zero4() { return uint4{0u, 0u, 0u, 0u}; }

__device__ __forceinline__ v8i make_op(uint4 a, uint4 b) {
  return v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

template <int FMT>
__device__ __forceinline__ v4f mma(const v8i& a, const v8i& b, int scale_a, int scale_b) {
  constexpr int f = FmtInfo<FMT>::kCode;
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, f, f, 0, scale_a, 0,
                                                          scale_b);
}

// Flip the sign of every e4m3 element of an operand (exact negation).
__device__ __forceinline__ v8i negate_fp8(const v8i& b, int mask) {
  return v8i{b[0] ^ mask, b[1] ^ mask, b[2] ^ mask, b[3] ^ mask,
             b[4] ^ mask, b[5] ^ mask, b[6] ^ mask, b[7] ^ mask};
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return min(max(x, lo), hi); }

__device__ __forceinline__ float neg_inf() { return __uint_as_float(kNegInfBits); }

__device__ __forceinline__ void store_nt(float* p, float v) { __builtin_nontemporal_store(v, p); }

// Raw buffer resources: the hardware range check drops stores and zero-fills
// loads whose VGPR offset is out of range, which keeps masking and ragged
// tails free of branches.  Ranges built here stay below kOOB bytes.
using Rsrc = __amdgpu_buffer_rsrc_t;
constexpr uint32_t kRsrcWord3 = 0x00020000u;      // gfx9 raw 32-bit buffer
constexpr int kOOB = 0x7ff00000;           // every range stays below this
constexpr int kNT = 2;                           // non-temporal cache hint

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, (int)kRsrcWord3);
}

// One operand from a buffer: 16 bytes at off_lo and 16 at off_hi (an offset
// of kOOB reads as zero).
__device__ __forceinline__ v8i buffer_operand(Rsrc r, int off_lo, int off_hi) {
  typedef int v4i __attribute__((ext_vector_type(4)));
  const v4i a = __builtin_amdgcn_raw_buffer_load_b128(r, off_lo, 0, 0);
  const v4i b = __builtin_amdgcn_raw_buffer_load_b128(r, off_hi, 0, 0);
  return v8i{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

__device__ __forceinline__ void buffer_store_nt(Rsrc r, int off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(v), r, off, 0, kNT);
}

// Per-wave state of the 4 query rows a wave owns: the A operands (Q) with
// their block scales, and this lane's weights.  H heads -> H/4 M tiles.
template <int FMT, int H, int D>
struct RowGroup {
  static constexpr int kMT = H / 4;
  static constexpr int kNKB = D / 32;                       // e8m0 blocks per row
  static constexpr int kRowBytes = OperandLayout<FMT, D>::kRowBytes;  // bytes per row

  v8i qa[kMT];
  int qs[kMT];
  float w[H];

  // a_row(r) = the query row that A row r (0..3 -> lanes' (l>>2)&3) reads;
  // e_row = the query row whose outputs this lane accumulates (lane >> 4).
  __device__ __forceinline__ void load(const uint8_t* __restrict__ q,
                                       const uint8_t* __restrict__ q_sf,
                                       const float* __restrict__ wts, int64_t a_row,
                                       int64_t e_row, int lane) {
    using L = OperandLayout<FMT, D>;
    const int g = lane >> 4;
    const int lo = L::lo(g), hi = L::hi(g);
    const int head_lo = lane & 3;
#pragma unroll
    for (int m = 0; m < kMT; ++m) {
      const int64_t hr = a_row * H + 4 * m + head_lo;
      const uint8_t* row = q + hr * L::kRowBytes;
      const uint4 a = lo >= 0 ? *reinterpret_cast<const uint4*>(row + lo) : zero4();
      const uint4 b = hi >= 0 ? *reinterpret_cast<const uint4*>(row + hi) : zero4();
      qa[m] = make_op(a, b);
      if constexpr (FmtInfo<FMT>::kMX) {
        qs[m] = L::scale_ok(g) ? (int)q_sf[hr * L::kBlocks + g] : 127;
      } else {
        qs[m] = 127;
      }
    }
    // The Q operands stay resident for the whole KV walk and are only read by
    // the MFMAs, which take A from AGPRs: keep them there and leave the VGPRs
    // to the accumulators, weights and streamed KV operands.
#pragma unroll
    for (int m = 0; m < kMT; ++m) asm volatile("" : "+a"(qa[m]));
    const float4* wp = reinterpret_cast<const float4*>(wts + e_row * H);
#pragma unroll
    for (int i = 0; i < H / 4; ++i) {
      float4 v = wp[i];
      w[4 * i + 0] = v.x;
      w[4 * i + 1] = v.y;
      w[4 * i + 2] = v.z;
      w[4 * i + 3] = v.w;
    }
  }

  // Software pipeline over 16-token steps.  acc holds the MFMA results of
  // the step being consumed; consume_and_issue() reduces them tile by tile
  // and, right behind each tile's VALU work, issues that tile's MFMA for the
  // next step into the same registers, so the matrix core runs the next
  // step while the VALU finishes this one.
  v4f acc[kMT];

  __device__ __forceinline__ void issue(const v8i& b, int scale_b) {
#pragma unroll
    for (int m = 0; m < kMT; ++m) acc[m] = mma<FMT>(qa[m], b, qs[m], scale_b);
  }

  // sum_h w[h] * max(S[h], 0) for this lane's (row, token) of the consumed
  // step; then acc <- the next step's products (operand b_next).
  __device__ __forceinline__ float consume_and_issue(const v8i& b_next, int scale_b) {
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
    for (int m = 0; m < kMT; ++m) {
      const v4f c = acc[m];
      s0 = __builtin_fmaf(w[4 * m + 0], __builtin_fmaxf(c[0], 0.f), s0);
      s1 = __builtin_fmaf(w[4 * m + 1], __builtin_fmaxf(c[1], 0.f), s1);
      s2 = __builtin_fmaf(w[4 * m + 2], __builtin_fmaxf(c[2], 0.f), s2);
      s3 = __builtin_fmaf(w[4 * m + 3], __builtin_fmaxf(c[3], 0.f), s3);
      acc[m] = mma<FMT>(qa[m], b_next, qs[m], scale_b);
      __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);   // 8 VALU
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // then 1 MFMA
    }
    return (s0 + s1) + (s2 + s3);
  }

  // The same reduction with no next step to issue.
  __device__ __forceinline__ float consume() const {
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
    for (int m = 0; m < kMT; ++m) {
      const v4f c = acc[m];
      s0 = __builtin_fmaf(w[4 * m + 0], __builtin_fmaxf(c[0], 0.f), s0);
      s1 = __builtin_fmaf(w[4 * m + 1], __builtin_fmaxf(c[1], 0.f), s1);
      s2 = __builtin_fmaf(w[4 * m + 2], __builtin_fmaxf(c[2], 0.f), s2);
      s3 = __builtin_fmaf(w[4 * m + 3], __builtin_fmaxf(c[3], 0.f), s3);
    }
    return (s0 + s1) + (s2 + s3);
  }

  // Non-pipelined: products and reduction of one step.
  __device__ __forceinline__ float weighted_relu_sum(const v8i& b, int scale_b) {
    issue(b, scale_b);
    return consume();
  }
};

// One streamed KV operand: the MFMA B operand of a 16-token step, its e8m0
// scale (MX) and its fp32 token scale (FP8).
struct KvOp {
  v8i b;
  int bs;
  float ks;
};

// Walk the 16-token steps from cl of one wave, software-pipelined: at the
// top of iteration j0 the accumulators hold the products of step j0 and the
// operand of step j0 + 16 has been in flight for two iterations.  The
// iteration reduces step j0 while issuing step j0 + 16's MFMAs, prefetches
// step j0 + 48, and hands (j0, value) to store(j0, v).  The three operand
// buffers rotate by name, three steps per trip, and the step count is padded
// to a multiple of three so the back-edge is the only branch (an exit inside
// the trip would let the compiler sink the next step's MFMAs behind it).
// load(j0, KvOp&) must zero-fill tokens past the KV range and store() must
// drop columns past the chunk.  Returns the first column not walked.
template <bool FLIP, class RG, class Load, class StoreFn>
__device__ __forceinline__ int compute_span(RG& rg, int cl, int ch, Load&& load, StoreFn&& store) {
  auto prep = [&](KvOp& o) {
    if constexpr (FLIP) o.b = negate_fp8(o.b, o.ks < 0.f ? (int)0x80808080 : 0);
  };
  const int steps = (ch - cl + kTileN - 1) / kTileN;
  const int end = cl + (steps + 2) / 3 * 3 * kTileN;
  KvOp o0, o1, o2;
  load(cl, o0);
  load(cl + kTileN, o1);
  load(cl + 2 * kTileN, o2);
  prep(o0);
  rg.issue(o0.b, o0.bs);
  float ks_prev = o0.ks;                       // token scale of the step in acc

  auto body = [&](int j0, KvOp& use, KvOp& ld) {
    const float ks_j0 = ks_prev;
    ks_prev = use.ks;
    load(j0 + 3 * kTileN, ld);                 // ld held step j0, already issued
    prep(use);
    float v = rg.consume_and_issue(use.b, use.bs);
    v *= __builtin_fabsf(ks_j0);
    asm volatile("" : "+v"(v));                // keep the reduction ahead of the store
    store(j0, v);
  };
  for (int j0 = cl; j0 < end; j0 += 3 * kTileN) {
    body(j0, o1, o0);
    body(j0 + kTileN, o2, o1);
    body(j0 + 2 * kTileN, o0, o2);
  }
  return end;
}

}  // namespace mqa
