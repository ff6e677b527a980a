// D = 64 on v_mfma_scale_f32_32x32x64_f8f6f4: the dense and compressed
// weighted-MQA-logits walk of one wave over 32-token steps.
//
// With D = 64 the 16x16x128 form of common.hpp carries zeros in half of K;
// the 32x32x64 form runs at the same rate per flop with none.  Operand and
// accumulator layout (measured on gfx950):
//   * A row / B column = lane % 32; lane group g = lane / 32 holds, for e4m3,
//     elements [16g, 16g+16) in dwords 0..3 and [32+16g, 32+16g+16) in dwords
//     4..7, for e2m1 elements [32g, 32g+32) in dwords 0..3; the e8m0 scale of
//     elements [32b, 32b+32) comes from lane group b;
//   * accumulator i of lane l is C[8 (i / 4) + 4 (l / 32) + i % 4][l % 32].
// Tile mapping: a wave owns 4 query rows; tile m = p * kHG + hg covers query
// pair p (rows 2p, 2p + 1) and heads [16 hg, 16 hg + 16).  A row r of the tile
// is query 2p + (r / 4) % 2, head 16 hg + 4 (r / 8) + r % 4, so the 16
// accumulators of lane l are the 16 heads of query 2p + l / 32 at token
// l % 32: the weighted ReLU head sum stays inside each lane, and each lane
// finishes two rows (queries l / 32 and 2 + l / 32) per step.
#pragma once

#include "common.hpp"

namespace mqa {

template <int FMT>
struct Layout32 {
  static constexpr int kRowBytes = FMT == kMXFP4 ? 32 : 64;
  static constexpr int kBlocks = 2;
  __device__ static constexpr int lo(int g) { return 16 * g; }
  __device__ static constexpr int hi(int g) { return FMT == kMXFP4 ? -1 : 32 + 16 * g; }
};

typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ v16f zero16() {
  v16f z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

template <int FMT>
__device__ __forceinline__ v16f mma32(const v8i& a, const v8i& b, int scale_a, int scale_b,
                                      v16f c) {
  constexpr int f = FmtInfo<FMT>::kCode;
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, f, f, 0, scale_a, 0, scale_b);
}

// The linear-half tile: A in e4m3 (the pieces of q'), B in the KV format.
template <int FMT>
__device__ __forceinline__ v16f mma32_lin(const v8i& a, const v8i& b, int scale_a, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, zero16(), 0, FmtInfo<FMT>::kCode, 0,
                                                         scale_a, 0, scale_b);
}

// LDS a wave needs to form the linear-half operand: partial sums fp32
// [4 queries][16 head lanes][64], piece codes [4][4 pieces][64] and their
// e8m0 scales [4][4][2].
struct LinLds32 {
  static constexpr int kPart = 0;
  static constexpr int kCodes = 4 * 16 * 64 * 4;
  static constexpr int kScales = kCodes + 4 * 4 * 64;
  static constexpr int kBytes = kScales + 4 * 4 * 2;
};

// Per-wave state of the 4 query rows row0 .. row0 + 3 (clamped to Sq - 1):
// the A operands (Q) of the 2 * kHG tiles with their block scales, and the
// weights of this lane's two rows.  LIN and EXACT as in RowGroup.
template <int FMT, int H, bool LIN, bool EXACT>
struct RowGroup32 {
  static_assert(!(LIN && EXACT), "the linear half rounds q' to e4m3 pieces");
  static constexpr int kTokens = 32;
  static constexpr int kHG = H < 16 ? 1 : H / 16;            // 16-head groups
  static constexpr int kMT = 2 * kHG;                        // tiles per step
  static constexpr int kWays = Split<FMT, EXACT>::kWays;
  using L = Layout32<FMT>;

  v8i qa[kMT];
  int qs[kMT];
  float w[2][16 * kHG];                                      // rows l/32 and 2 + l/32; 0 past H
  v8i ql;
  int qls;
  // LIN, until the linear-half operand is formed: w / 2 of the (row, head)
  // of this lane's A row of tile m, and (MXFP8) that head's two block scales.
  float wl[kMT];
  int wsf[kMT];

  // Row (within the wave's 4) and head that A row l % 32 of tile m reads.
  __device__ static __forceinline__ int a_of(int lane, int m) {
    return 2 * (m / kHG) + ((lane >> 2) & 1);
  }
  __device__ static __forceinline__ int head_of(int lane, int m) {
    return 16 * (m % kHG) + 4 * ((lane >> 3) & 3) + (lane & 3);
  }

  // Issues the loads of the Q operands, their block scales and the weights
  // (LIN: also the weight and block scales make_lin takes for each of this
  // lane's A rows, so that forming q' waits for no further load); finish()
  // then forms the linear-half operand and pins the operands.
  __device__ __forceinline__ void load(const uint8_t* __restrict__ q,
                                       const uint8_t* __restrict__ q_sf,
                                       const void* __restrict__ wts, bool w_bf16, int row0, int sq,
                                       int lane) {
    const int g = lane >> 5;
#pragma unroll
    for (int m = 0; m < kMT; ++m) {
      const int64_t row = min(row0 + a_of(lane, m), sq - 1);
      const int head = head_of(lane, m);
      uint4 a = zero4(), b = zero4();
      qs[m] = 127;
      wl[m] = 0.f;
      wsf[m] = 127 | (127 << 8);
      if (head < H) {
        const int64_t hr = row * H + head;
        const uint8_t* src = q + hr * L::kRowBytes;
        a = *reinterpret_cast<const uint4*>(src + L::lo(g));
        if constexpr (L::hi(0) >= 0) b = *reinterpret_cast<const uint4*>(src + L::hi(g));
        if constexpr (FmtInfo<FMT>::kMX) qs[m] = (int)q_sf[hr * L::kBlocks + g];
        if constexpr (LIN) {
          wl[m] = 0.5f * (w_bf16 ? bf16_value(static_cast<const uint16_t*>(wts)[hr])
                                 : static_cast<const float*>(wts)[hr]);
          if constexpr (FmtInfo<FMT>::kMX && FMT != kMXFP4)
            wsf[m] = (int)*reinterpret_cast<const uint16_t*>(q_sf + hr * L::kBlocks);
        }
      }
      qa[m] = make_op(a, b);
    }
    constexpr float kW = LIN ? 0.5f : 1.f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int64_t e = min(row0 + 2 * k + (lane >> 5), sq - 1);
#pragma unroll
      for (int i = 0; i < 16 * kHG; i += 4) {
        if (i < H) {
          if (w_bf16) {
            const uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(wts) +
                                                            e * H + i);
            w[k][i + 0] = kW * bf16_value(v.x & 0xffffu);
            w[k][i + 1] = kW * bf16_value(v.x >> 16);
            w[k][i + 2] = kW * bf16_value(v.y & 0xffffu);
            w[k][i + 3] = kW * bf16_value(v.y >> 16);
          } else {
            const float4 v =
                *reinterpret_cast<const float4*>(static_cast<const float*>(wts) + e * H + i);
            w[k][i + 0] = kW * v.x;
            w[k][i + 1] = kW * v.y;
            w[k][i + 2] = kW * v.z;
            w[k][i + 3] = kW * v.w;
          }
        } else {
          w[k][i + 0] = w[k][i + 1] = w[k][i + 2] = w[k][i + 3] = 0.f;
        }
      }
    }
  }

  // The Q operands stay resident for the whole walk and are only read by the
  // MFMAs, which take A from AGPRs: pin them there (LIN: after forming the
  // linear-half operand from them).
  __device__ __forceinline__ void finish(int lane, char* lin_lds) {
    if constexpr (LIN) make_lin(lane, lin_lds);
#pragma unroll
    for (int m = 0; m < kMT; ++m) asm volatile("" : "+a"(qa[m]));
    if constexpr (LIN) asm volatile("" : "+a"(ql));
  }

  // LIN: the linear-half operand (RowGroup::make_lin's arithmetic in this
  // layout).  1. each lane sums, for its two queries, the elements it holds
  // over its kHG heads (head lane 4 ((l/8) % 4) + l % 4 of each 16-head
  // group) and writes the partial sums; 2. lane L adds the 16 head lanes'
  // partials of 4 consecutive elements of query L / 16 (fixed order) and
  // splits them into four e4m3 pieces with e8m0 block scales; 3. lane l reads
  // its operand of the linear tile, A row r = l % 32 = (query 2 ((r/8) % 2) +
  // (r/4) % 2, piece r % 4) for r < 16, zero rows above.  The LDS traffic stays
  // within the wave (in-order LDS access).
  __device__ __forceinline__ void make_lin(int lane, char* lds) {
    constexpr bool kFP4 = FMT == kMXFP4;
    constexpr int kD = 64;
    const int g = lane >> 5;
    const int hl = 4 * ((lane >> 3) & 3) + (lane & 3);
    const int e_lo = kFP4 ? 32 * g : L::lo(g);                // elements of slots [0, 16 or 32)
    const int e_hi = L::hi(g);                                // e4m3: of slots [16, 32)
    float* part = reinterpret_cast<float*>(lds + LinLds32::kPart);
    typedef float v2f_ __attribute__((ext_vector_type(2)));

#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int a = 2 * p + ((lane >> 2) & 1);
      float acc[32];
#pragma unroll
      for (int k = 0; k < 32; ++k) acc[k] = 0.f;
#pragma unroll
      for (int hg = 0; hg < kHG; ++hg) {
        const int m = p * kHG + hg;
        const int head = 16 * hg + hl;
        if (head >= H) continue;
        const float wv = wl[m];
        float w_lo = wv, w_hi = wv;
        if constexpr (kFP4) {
          w_lo = ldexpf(wv, qs[m] - 127);             // block g's scale is this lane's operand's
        } else if constexpr (FmtInfo<FMT>::kMX) {
          // elements [16g, 16g + 16) lie in block 0, [32 + 16g, 48 + 16g) in block 1
          w_lo = ldexpf(wv, (wsf[m] & 0xff) - 127);
          w_hi = ldexpf(wv, (wsf[m] >> 8) - 127);
        }
        if constexpr (kFP4) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t word = (uint32_t)qa[m][j];
            const v2f_ v[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 0),
                               __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 1),
                               __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 2),
                               __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 3)};
#pragma unroll
            for (int sel = 0; sel < 4; ++sel) {
              acc[8 * j + 2 * sel] = __builtin_fmaf(w_lo, v[sel][0], acc[8 * j + 2 * sel]);
              acc[8 * j + 2 * sel + 1] = __builtin_fmaf(w_lo, v[sel][1], acc[8 * j + 2 * sel + 1]);
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const uint32_t word = (uint32_t)qa[m][j];
            const float wj = j < 4 ? w_lo : w_hi;
            const v2f_ x = __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
            const v2f_ y = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);
            acc[4 * j + 0] = __builtin_fmaf(wj, x[0], acc[4 * j + 0]);
            acc[4 * j + 1] = __builtin_fmaf(wj, x[1], acc[4 * j + 1]);
            acc[4 * j + 2] = __builtin_fmaf(wj, y[0], acc[4 * j + 2]);
            acc[4 * j + 3] = __builtin_fmaf(wj, y[1], acc[4 * j + 3]);
          }
        }
      }
      float* dst = part + (a * 16 + hl) * kD;
#pragma unroll
      for (int k = 0; k < 32; k += 4) {
        const int e = (kFP4 || k < 16) ? e_lo + k : e_hi + (k - 16);
        *reinterpret_cast<float4*>(dst + e) = float4{acc[k], acc[k + 1], acc[k + 2], acc[k + 3]};
      }
    }
    asm volatile("" ::: "memory");

    // 2. the pieces of elements [e0, e0 + 4) of query qq = lane / 16
    constexpr int kLanesPerBlock = 8;                        // 32 elements, 4 per lane
    const int qq = lane >> 4, e0 = 4 * (lane & 15);
    float r[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < 16; ++h) {
      const float4 v = *reinterpret_cast<const float4*>(part + (qq * 16 + h) * kD + e0);
      r[0] += v.x;
      r[1] += v.y;
      r[2] += v.z;
      r[3] += v.w;
    }
    uint8_t* codes = reinterpret_cast<uint8_t*>(lds + LinLds32::kCodes);
    uint8_t* scales = reinterpret_cast<uint8_t*>(lds + LinLds32::kScales);
#pragma unroll
    for (int pc = 0; pc < 4; ++pc) {
      float mx = __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(r[0]), __builtin_fabsf(r[1])),
                                 __builtin_fmaxf(__builtin_fabsf(r[2]), __builtin_fabsf(r[3])));
#pragma unroll
      for (int o = 1; o < kLanesPerBlock; o <<= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, o));
      int sc = -127;
      if (mx > 0.f) {
        int e;
        const float f = frexpf(mx, &e);                      // mx / 2^sc <= 448 = 0.875 * 2^9
        sc = min(max(f <= 0.875f ? e - 9 : e - 8, -127), 127);
      }
      const int lo2 = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(r[0], -sc), ldexpf(r[1], -sc), 0, false);
      const uint32_t word = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(r[2], -sc),
                                                                      ldexpf(r[3], -sc), lo2, true);
      const v2f_ x = __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
      const v2f_ y = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);
      r[0] -= ldexpf(x[0], sc);
      r[1] -= ldexpf(x[1], sc);
      r[2] -= ldexpf(y[0], sc);
      r[3] -= ldexpf(y[1], sc);
      *reinterpret_cast<uint32_t*>(codes + (qq * 4 + pc) * kD + e0) = word;
      if ((lane & (kLanesPerBlock - 1)) == 0)
        scales[(qq * 4 + pc) * 2 + e0 / 32] = (uint8_t)(sc + 127);
    }
    asm volatile("" ::: "memory");

    // 3. this lane's operand of the linear tile
    const int rr = lane & 31;
    ql = make_op(zero4(), zero4());
    qls = 127;
    if (rr < 16) {
      const int query = 2 * ((rr >> 3) & 1) + ((rr >> 2) & 1), piece = rr & 3;
      const uint8_t* prow = codes + (query * 4 + piece) * kD;
      ql = make_op(*reinterpret_cast<const uint4*>(prow + 16 * g),
                   *reinterpret_cast<const uint4*>(prow + 32 + 16 * g));
      qls = (int)scales[(query * 4 + piece) * 2 + g];
    }
  }

  // Pipeline as in RowGroup: tile m of a step lands in acc[m % kRing] and the
  // VALU reduces the tile kLag slots behind the MFMA being issued.  s[k][.]
  // are four running partial sums of row k (rows l/32 and 2 + l/32).
  // (EXACT keeps two tiles in flight: its eight KV operand copies and two
  // rows of weights leave no room for four.)
  static constexpr int kRing = kMT < 4 ? kMT : (EXACT ? 2 : 4);
  static constexpr int kLag = kRing / 2;
  static constexpr int kValuPerTile = LIN ? 16 : 32;
  v16f acc[kRing];
  float s[2][4];

  __device__ __forceinline__ void start() {
#pragma unroll
    for (int r = 0; r < kRing; ++r) acc[r] = zero16();
#pragma unroll
    for (int i = 0; i < 4; ++i) s[0][i] = s[1][i] = 0.f;
  }

  __device__ __forceinline__ void reduce_tile(int mc, const v16f& c) {
    const int p = mc / kHG, hg = mc % kHG;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float r = LIN ? __builtin_fabsf(c[i]) : __builtin_fmaxf(c[i], 0.f);
      s[p][i & 3] = __builtin_fmaf(w[p][16 * hg + i], r, s[p][i & 3]);
    }
  }

  // The finished step's two totals; the sums restart from the next step's
  // linear tile (accumulators 0..3: row l/32's pieces, 4..7: row 2 + l/32's).
  __device__ __forceinline__ float2 take(const v16f& next_lin) {
    const float2 v = {(s[0][0] + s[0][1]) + (s[0][2] + s[0][3]),
                      (s[1][0] + s[1][1]) + (s[1][2] + s[1][3])};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[0][i] = LIN ? next_lin[i] : 0.f;
      s[1][i] = LIN ? next_lin[4 + i] : 0.f;
    }
    return v;
  }

  template <class Done>
  __device__ __forceinline__ void step(const v8i& b, int scale_b, Done&& done) {
    v16f lin = zero16();
    if constexpr (LIN) {
      lin = mma32_lin<FMT>(ql, b, qls, scale_b);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    // EXACT with several head groups: each tile forms its eight KV copies from
    // an opaque copy of b, so they live for one tile only (two rows of
    // weights and eight copies held across the step exceed the VGPRs).
    constexpr bool kCopyPerTile = kWays > 1 && kHG > 1;
    v8i bp[kWays];
    if constexpr (!kCopyPerTile) {
#pragma unroll
      for (int k = 0; k < kWays; ++k) bp[k] = Split<FMT, EXACT>::part(b, k);
    }
#pragma unroll
    for (int m = 0; m < kMT; ++m) {
      reduce_tile((m - kLag + kMT) % kMT, acc[(m - kLag + kRing) % kRing]);
      if constexpr (kCopyPerTile) {
        v8i bm = b;
        asm volatile("" : "+v"(bm));
#pragma unroll
        for (int k = 0; k < kWays; ++k) bp[k] = Split<FMT, EXACT>::part(bm, k);
      }
      v16f c = mma32<FMT>(qa[m], bp[0], qs[m], scale_b, zero16());
#pragma unroll
      for (int k = 1; k < kWays; ++k) c = mma32<FMT>(qa[m], bp[k], qs[m], scale_b, c);
      acc[m % kRing] = c;
      __builtin_amdgcn_sched_group_barrier(0x002, kValuPerTile, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, kWays, 0);
      if (m == kLag - 1) done(take(lin));
    }
  }

  __device__ __forceinline__ float2 drain() {
#pragma unroll
    for (int k = 0; k < kLag; ++k) reduce_tile(kMT - kLag + k, acc[(kMT - kLag + k) % kRing]);
    return take(zero16());
  }
};

constexpr int kTripCols32 = 32 * kKvStages;                  // columns per trip
static_assert(kTripCols32 == 128, "StagedSink32::buffer() divides by 128");

// Clean output of the 32-token walk.  A trip's 4 rows x 128 columns are staged
// in LDS; lane l reads back row l / 16, columns 8 (l % 16) .. +7 and stores
// them as two 16-byte groups (512-byte runs per row).  Each group is stored
// iff it lies in the wave's columns (at or below last_j0, see trip()).
template <int OUT>
struct StagedSink32 {
  float* stage;              // 2 x [4][128] floats in LDS
  Rsrc r;
  int base;                  // first column of the walk
  int put0, put1;            // this lane's slots of rows l/32 and 2 + l/32, column l % 32
  int rd_idx;                // this lane's read-back group: row l / 16, column 8 (l % 16)
  int row_off;               // byte offset of that group in the output at column 0
  int last_j0;               // half k of trip j0's group is stored iff base <= j0, j0 + 4k <= last_j0
  int rel0, len0, rel1, len1;  // column j0 + l%32 of row k is in range iff j0 + rel_k in [0, len_k)
  float4 pa, pb;             // the last trip read back, and its store offsets
  int off_a, off_b;

  __device__ __forceinline__ float* buffer(int j0) const {
    return stage + (((j0 - base) >> 7) & 1) * (kRowsPerWave * kTripCols32);
  }
  __device__ __forceinline__ void put(int u, int j0, float2 v) {
    float* b = buffer(j0);
    b[put0 + u * 32] = (uint32_t)(j0 + rel0) < (uint32_t)len0 ? v.x : neg_inf();
    b[put1 + u * 32] = (uint32_t)(j0 + rel1) < (uint32_t)len1 ? v.y : neg_inf();
    if (u == 0) {
      OutElem<OUT>::store4(r, off_a, pa);
      OutElem<OUT>::store4(r, off_b, pb);
    }
  }
  __device__ __forceinline__ void trip(int jt) {
    asm volatile("" ::: "memory");
    pa = *reinterpret_cast<const float4*>(buffer(jt) + rd_idx);
    pb = *reinterpret_cast<const float4*>(buffer(jt) + rd_idx + 4);
    const int early = oob_if(jt < base);
    off_a = (jt <= last_j0 ? row_off + OutElem<OUT>::kBytes * jt : kOOB) | early;
    off_b = (jt + 4 <= last_j0 ? row_off + OutElem<OUT>::kBytes * (jt + 4) : kOOB) | early;
    asm volatile("" ::: "memory");
  }
  __device__ __forceinline__ void finish() {
    OutElem<OUT>::store4(r, off_a, pa);
    OutElem<OUT>::store4(r, off_b, pb);
  }
};

// Keep and compressed: each in-range value straight to its column.
template <int OUT, class OffFn>
struct DwordSink32 {
  Rsrc r;
  OffFn off;                 // (k, j0) -> byte offset of row k's value, or kOOB
  int lo_j0;                 // steps below lo_j0 are dropped
  __device__ __forceinline__ void put(int, int j0, float2 v) {
    const int early = oob_if(j0 < lo_j0);
    OutElem<OUT>::store1(r, off(0, j0) | early, v.x);
    OutElem<OUT>::store1(r, off(1, j0) | early, v.y);
  }
  __device__ __forceinline__ void trip(int) {}
  __device__ __forceinline__ void finish() {}
};

// Arithmetic of a D = 64 instance: EXACT as in DenseMode; the linear half for
// H >= 32 (the per-lane epilogue of this layout is 16 heads per accumulator
// tile, so it pays off from two head groups on).
template <int H, bool EXACT>
struct DenseMode32 {
  static constexpr bool kExact = EXACT || H <= 16;
  static constexpr bool kLin = H >= 32 && !kExact;
};

// One wave's piece of row group row0 / 4 for D = 64: dense_group's contract
// (dense_kernel.hpp) in the 32x32x64 tiles.  Lane l computes rows l / 32 and
// 2 + l / 32 of the group at column l % 32 of each 32-token step.
template <int FMT, int STORE, int OUT, bool EXACT, int H, class SegFn>
__device__ __forceinline__ void dense_group32(const DenseParams& p, int row0, int wave, int lane,
                                              SegFn&& seg) {
  using M = DenseMode32<H, EXACT>;
  using RG = RowGroup32<FMT, H, M::kLin, M::kExact>;
  using L = Layout32<FMT>;
  using OE = OutElem<OUT>;
  constexpr int kRowBytes = L::kRowBytes;
  constexpr int kOB = OE::kBytes;

  const int h = lane >> 5;                       // this lane's rows: h and 2 + h
  const int n = lane & 31;                       // its column in a 32-token step

  int ks_raw[kRowsPerWave], ke_raw[kRowsPerWave];
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) {
    const int rr = min(row0 + r, p.sq - 1);
    ks_raw[r] = p.k_start[rr];
    ke_raw[r] = p.k_end[rr];
  }
  __builtin_amdgcn_sched_barrier(0);

  RG rg;
  char* lin_lds = nullptr;
  if constexpr (M::kLin) {
    __shared__ __attribute__((aligned(16))) char lin_all[kDenseWaves][LinLds32::kBytes];
    lin_lds = lin_all[wave];
  }

  // The Q operands and weights do not depend on the ranges: they go out while
  // the ranges' (scalar) loads are in flight.
  rg.load(p.q, p.q_sf, p.w, p.w_bf16 != 0, row0, p.sq, lane);
  __builtin_amdgcn_sched_barrier(0);

  int s_r[kRowsPerWave], e_r[kRowsPerWave];
  int lo = 0x7fffffff, hi = 0;
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) {
    s_r[r] = clampi(ks_raw[r], 0, p.skv);
    e_r[r] = row0 + r < p.sq ? clampi(ke_raw[r], s_r[r], p.skv) : s_r[r];
    if (e_r[r] > s_r[r]) {
      lo = min(lo, s_r[r]);
      hi = max(hi, e_r[r]);
    }
  }
  const int sA = h == 0 ? s_r[0] : s_r[1], eA = h == 0 ? e_r[0] : e_r[1];   // row h
  const int sB = h == 0 ? s_r[2] : s_r[3], eB = h == 0 ? e_r[2] : e_r[3];   // row 2 + h

  const int lo64 = lo < hi ? (lo & ~(kTripCols - 1)) : 0;
  const GroupSeg sg = seg(group_trips(lo, hi));
  const int b0 = min(lo64 + (int)min((int64_t)sg.t_a * kTripCols, (int64_t)p.skv), p.skv);
  const int b1 = min(lo64 + (int)min((int64_t)sg.t_b * kTripCols, (int64_t)p.skv), p.skv);
  const int c0 = sg.first ? 0 : b0;
  const int c1 = sg.last ? p.skv : b1;
  int cl = b0, ch = min(b1, hi);
  if (cl >= ch) { cl = c1; ch = c1; }
  const int lenA = max(0, min(eA, c1) - sA), relA = n - sA;
  const int lenB = max(0, min(eB, c1) - sB), relB = n - sB;

  // KV operand of lane l: token j0 + l % 32, lane group l / 32's pieces and
  // block scale.
  const int g = lane >> 5;
  const Rsrc kv_r = make_rsrc(p.kv, (uint32_t)((int64_t)p.skv * kRowBytes));
  const int b_lo = n * kRowBytes + L::lo(g);
  const int b_hi = L::hi(g) >= 0 ? n * kRowBytes + L::hi(g) : kOOB;
  Rsrc sc_r;
  int sc_lane;
  if constexpr (FmtInfo<FMT>::kMX) {
    sc_r = make_rsrc(p.kv_sf, (uint32_t)((int64_t)p.skv * L::kBlocks));
    sc_lane = n * L::kBlocks + g;
  } else {
    sc_r = make_rsrc(p.kv_scale, (uint32_t)((int64_t)p.skv * 4));
    sc_lane = 4 * n;
  }
  auto load_b = [&](int j0, KvOp& o) {
    o.b = buffer_operand(kv_r, b_lo, b_hi, j0 * kRowBytes);
    if constexpr (FmtInfo<FMT>::kMX) {
      o.bs = __builtin_amdgcn_raw_buffer_load_b8(sc_r, sc_lane, j0 * L::kBlocks, 0);
      o.ks = 1.f;
    } else {
      o.bs = 127;
      o.ks = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(sc_r, sc_lane, 4 * j0, 0));
    }
  };

  // The walk's first operands and the first round of the scale scan below go
  // out next; the linear-half operand is formed from the Q operands while
  // they are in flight.
  KvOp ring[kKvStages];
  if (cl < ch) prefetch_span<32>(cl, ring, load_b);

  // For FP8, whether any token scale of the span is negative (the FLIP walk
  // then negates those tokens' codes; ReLU(s x) = |s| ReLU(sign(s) x)):
  // 16-byte loads, kPer in flight per lane, zero past the array.
  typedef int v4i __attribute__((ext_vector_type(4)));
  constexpr int kPer = 8;
  constexpr int kScanRound = 4 * kPer * kWaveLanes;          // columns per round
  v4i sv[kPer];
  if constexpr (!FmtInfo<FMT>::kMX) {
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      sv[u] = __builtin_amdgcn_raw_buffer_load_b128(sc_r, 4 * (cl + 4 * lane + 4 * kWaveLanes * u), 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);

  rg.finish(lane, lin_lds);
  __builtin_amdgcn_sched_barrier(0);

  bool flip = false;
  if constexpr (!FmtInfo<FMT>::kMX) {
    int neg = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) neg |= (sv[u][0] | sv[u][1]) | (sv[u][2] | sv[u][3]);
    for (int j = cl + kScanRound + 4 * lane; j < ch; j += kScanRound) {
#pragma unroll
      for (int u = 0; u < kPer; ++u)
        sv[u] = __builtin_amdgcn_raw_buffer_load_b128(sc_r, 4 * (j + 4 * kWaveLanes * u), 0, 0);
#pragma unroll
      for (int u = 0; u < kPer; ++u) neg |= (sv[u][0] | sv[u][1]) | (sv[u][2] | sv[u][3]);
    }
    // any sign bit set (-0.0 is harmless; scales past the span only cost the
    // exact path)
    flip = cl < ch && __ballot(neg < 0) != 0;
  }

  Rsrc out_r;
  char* const out_base = static_cast<char*>(p.out);
  int64_t first = 0;
  if constexpr (STORE == kCompressed) {
    first = uniform64(p.row_off[row0]);
    const int64_t last = uniform64(p.row_off[min(row0 + kRowsPerWave, p.sq)]);
    out_r = make_rsrc(out_base + first * kOB, (uint32_t)((last - first) * kOB));
  } else {
    const int rows = min(kRowsPerWave, p.sq - row0);
    out_r = make_rsrc(out_base + (int64_t)row0 * p.stride * kOB, (uint32_t)(rows * p.stride * kOB));
  }

  auto walk = [&](auto& sink) {
    int walked = ch;
    if (cl < ch) {
      if (flip) walked = compute_span<true>(rg, cl, ch, ring, load_b, sink);
      else walked = compute_span<false>(rg, cl, ch, ring, load_b, sink);
    }
    return walked;
  };

  if constexpr (STORE == kDenseClean) {
    __shared__ __attribute__((aligned(16))) float stage_all[kDenseWaves][2 * kRowsPerWave * kTripCols32];
    float* stage = stage_all[wave];
    const int rows = min(kRowsPerWave, p.sq - row0);
    const int rg_row = lane >> 4;                // read-back group: row, 8 columns from col8
    const int col8 = 8 * (lane & 15);
    const bool grp_ok = rg_row < rows;
    const int grp_off = (int)(rg_row * p.stride * kOB) + kOB * col8;
    const int lim = c1 & ~3;
    const float4 ninf4 = {neg_inf(), neg_inf(), neg_inf(), neg_inf()};
    const int last_j0 = grp_ok ? lim - col8 - 4 : -0x40000000;
    // -inf over columns [from, to) (from a multiple of 64): the lane's two
    // 4-column halves of each 128-column trip, each only when inside.
    auto fill = [&](int from, int to) {
      const int lim_to = min(to, lim);
      for (int j0 = from; j0 < to; j0 += kTripCols32) {
        const int ca = j0 + col8;
        OE::store4(out_r, (grp_ok && ca + 4 <= lim_to) ? grp_off + kOB * j0 : kOOB, ninf4);
        OE::store4(out_r, (grp_ok && ca + 8 <= lim_to) ? grp_off + kOB * (j0 + 4) : kOOB, ninf4);
      }
    };
    fill(c0, cl);
    StagedSink32<OUT> sink{stage, out_r, cl, h * kTripCols32 + n, (2 + h) * kTripCols32 + n,
                           rg_row * kTripCols32 + col8, grp_off, last_j0, relA, lenA, relB, lenB,
                           ninf4, ninf4, kOOB, kOOB};
    const int walked = walk(sink);
    fill(cl < ch ? walked : c1, c1);
    // The last 1..3 columns of a row whose width is not a multiple of 4, one
    // per lane (row l / 16), from the last trip's LDS buffer or -inf.
    if ((c1 & 3) != 0) {
      const int gs = c1 & ~3;
      const int tr = lane >> 4, tc = lane & 15;
      if (tr < rows && gs + tc < c1) {
        float v = neg_inf();
        const int jt = walked - kTripCols32;
        if (cl < ch && gs >= jt && gs < walked) v = sink.buffer(jt)[tr * kTripCols32 + (gs - jt) + tc];
        OE::store1(out_r, (int)(tr * p.stride * kOB) + kOB * (gs + tc), v);
      }
    }
  } else {
    int off0 = 0, off1 = 0;                      // byte offsets of (row, column 0 of the step)
    if constexpr (STORE == kCompressed) {
      const bool okA = row0 + h < p.sq, okB = row0 + 2 + h < p.sq;
      off0 = okA ? (int)((p.row_off[min(row0 + h, p.sq - 1)] - first - sA) * kOB) : 0;
      off1 = okB ? (int)((p.row_off[min(row0 + 2 + h, p.sq - 1)] - first - sB) * kOB) : 0;
    } else {
      off0 = (int)(h * p.stride * kOB);
      off1 = (int)((2 + h) * p.stride * kOB);
    }
    off0 += kOB * n;
    off1 += kOB * n;
    auto off = [&](int k, int j0) {
      const bool in = k == 0 ? (uint32_t)(j0 + relA) < (uint32_t)lenA
                             : (uint32_t)(j0 + relB) < (uint32_t)lenB;
      return in ? (k == 0 ? off0 : off1) + kOB * j0 : kOOB;
    };
    DwordSink32<OUT, decltype(off)> sink{out_r, off, cl};
    walk(sink);
  }
}

}  // namespace mqa
