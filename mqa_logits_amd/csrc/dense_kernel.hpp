// Dense and compressed weighted MQA logits for gfx950: the kernel templates
// and their instance dispatch (instantiated per logits type and work split in
// dense.hip, dense_bf16.hip, dense_sched.hip and dense_sched_bf16.hip).
//
//   logits[i, j] = sum_h w[i, h] * ReLU(kv_scale[j] * <q[i, h, :], kv[j, :]>)
//
// for s_i <= j < e_i, -inf elsewhere (dense clean), untouched elsewhere (dense
// keep), or packed by row offsets (compressed) -- the math-warp reduction,
// compressed-logits store and clean fill described in "How to Implement MQA
// (Multi-Query Attention) Logits Computation with DeepGEMM" (Core
// Architecture Components) and "[PR #435] Improve SM100 MX MQA logits
// clean-output performance" (Description).
//
// Work split: a wave owns 4 consecutive query rows and a run of KV columns,
// keeps the rows' Q operands and weights in registers and walks the run 16
// tokens at a time.  Without a schedule, the 4 waves of a block take 4
// consecutive row groups and the same chunk of their columns; with one, each
// wave walks its piece of an even split of all groups' trips.  Tokens outside
// the union of a group's row ranges are -inf fill (no MFMA); tokens inside
// are computed and masked per row in the same store.  No second pass, no
// atomics: each output element is written by exactly one lane.
#pragma once

#include "common.hpp"
#include "launch.hpp"
#include "tile32.hpp"

namespace mqa {

constexpr int kDenseThreads = kWaveLanes * kDenseWaves;

// Arithmetic of an instance: EXACT splits the KV operand so that every
// product reaches the accumulator exactly (always for H <= 16, whose few
// heads leave the tolerance too little room for the matrix core's grouped
// summation; on request otherwise); LIN takes ReLU's linear half from the
// weighted query sum (H = 64, not EXACT: the sum is rounded to e4m3 pieces).
template <int H, bool EXACT>
struct DenseMode {
  static constexpr bool kExact = EXACT || H <= 16;
  static constexpr bool kLin = H == kLinHeads && !kExact;
};

// One wave's piece of row group row0 / 4; seg(trips) -> GroupSeg picks it.
template <int FMT, int H, int D, int STORE, int OUT, bool EXACT, class SegFn>
__device__ __forceinline__ void dense_group(const DenseParams& p, int row0, int wave, int lane,
                                            SegFn&& seg) {
  using M = DenseMode<H, EXACT>;
  using RG = RowGroup<FMT, H, D, M::kLin, M::kExact>;
  using L = OperandLayout<FMT, D>;
  using OE = OutElem<OUT>;
  constexpr int kNKB = RG::kNKB;
  constexpr int kRowBytes = RG::kRowBytes;
  constexpr int kOB = OE::kBytes;              // bytes per logits element

  // ---- this wave's 4 rows ----------------------------------------------
  const int g = lane >> 4;                     // output row of this lane
  const int n = lane & 15;                     // output column in a 16-token tile
  const int e_row = row0 + g;
  const bool row_ok = e_row < p.sq;
  const int e_row_c = min(e_row, p.sq - 1);
  const int a_row_c = min(row0 + ((lane >> 2) & 3), p.sq - 1);

  // The 4 rows' ranges (wave-uniform loads) go out first: the column split
  // needs them, and in-order load completion would otherwise make them wait
  // for the Q operands, the largest loads of the prologue.
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
    __shared__ __attribute__((aligned(16))) char lin_all[kDenseWaves][LinLds<D>::kBytes];
    lin_lds = lin_all[wave];
  }
  rg.load(p.q, p.q_sf, p.w, p.w_bf16 != 0, a_row_c, e_row_c, lane, H, 0, lin_lds);
  __builtin_amdgcn_sched_barrier(0);

  // The ranges, their union, and this lane's row.
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
  const int s_row = g == 0 ? s_r[0] : g == 1 ? s_r[1] : g == 2 ? s_r[2] : s_r[3];
  const int e_end = g == 0 ? e_r[0] : g == 1 ? e_r[1] : g == 2 ? e_r[2] : e_r[3];

  // This wave computes trips [t_a, t_b) of the union, i.e. columns [cl, ch),
  // and owns the output columns [c0, c1) around them.
  const int lo64 = lo < hi ? (lo & ~(kTripCols - 1)) : 0;
  const GroupSeg sg = seg(group_trips(lo, hi));
  const int b0 = min(lo64 + (int)min((int64_t)sg.t_a * kTripCols, (int64_t)p.skv), p.skv);
  const int b1 = min(lo64 + (int)min((int64_t)sg.t_b * kTripCols, (int64_t)p.skv), p.skv);
  const int c0 = sg.first ? 0 : b0;
  const int c1 = sg.last ? p.skv : b1;
  int cl = b0, ch = min(b1, hi);
  if (cl >= ch) { cl = c1; ch = c1; }          // nothing to compute in this piece
  const int len = max(0, min(e_end, c1) - s_row);
  const int rel_n = n - s_row;                 // (j0 + rel_n) in [0, len) iff in range

  // ---- output addressing: one buffer resource per wave -------------------
  Rsrc out_r;
  int lane_off;                                // byte offset of (row g, column n), column 0
  char* const out_base = static_cast<char*>(p.out);
  if constexpr (STORE == kCompressed) {
    const int64_t first = uniform64(p.row_off[row0]);
    const int64_t last = uniform64(p.row_off[min(row0 + kRowsPerWave, p.sq)]);
    out_r = make_rsrc(out_base + first * kOB, (uint32_t)((last - first) * kOB));
    lane_off = (int)(row_ok ? (p.row_off[e_row_c] - first - s_row) * kOB : 0) + kOB * n;
  } else {
    const int rows = min(kRowsPerWave, p.sq - row0);
    out_r = make_rsrc(out_base + (int64_t)row0 * p.stride * kOB, (uint32_t)(rows * p.stride * kOB));
    lane_off = (int)(g * p.stride * kOB) + kOB * n;
  }

  // ---- KV operands ---------------------------------------------------------
  // KV operand of lane l: token j0 + l % 16, the two 16-byte pieces of lane
  // group l / 16 (OperandLayout), and that group's e8m0 block scale (MX).
  const int kb = lane >> 4;
  const bool kb_ok = L::scale_ok(kb);
  const Rsrc kv_r = make_rsrc(p.kv, (uint32_t)((int64_t)p.skv * kRowBytes));
  const int b_lo = L::lo(kb) >= 0 ? n * kRowBytes + L::lo(kb) : kOOB;
  const int b_hi = L::hi(kb) >= 0 ? n * kRowBytes + L::hi(kb) : kOOB;
  Rsrc sc_r;
  int sc_lane;
  if constexpr (FmtInfo<FMT>::kMX) {
    sc_r = make_rsrc(p.kv_sf, (uint32_t)((int64_t)p.skv * kNKB));
    sc_lane = kb_ok ? n * kNKB + kb : kOOB;
  } else {
    sc_r = make_rsrc(p.kv_scale, (uint32_t)((int64_t)p.skv * 4));
    sc_lane = 4 * n;
  }

  // operand, e8m0 scale (MX) and fp32 token scale (FP8) of step j0; tokens
  // past Skv read as zero.
  auto load_b = [&](int j0, KvOp& o) {
    o.b = buffer_operand(kv_r, b_lo, b_hi, j0 * kRowBytes);
    if constexpr (FmtInfo<FMT>::kMX) {
      o.bs = kb_ok ? __builtin_amdgcn_raw_buffer_load_b8(sc_r, sc_lane, j0 * kNKB, 0) : (uint8_t)127;
      o.ks = 1.f;
    } else {
      o.bs = 127;
      o.ks = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(sc_r, sc_lane, 4 * j0, 0));
    }
  };

  // The walk's first operands go out before the scale scan below, so both
  // latencies overlap (and that of the Q loads above).
  KvOp ring[kKvStages];
  if (cl < ch) prefetch_span(cl, ring, load_b);

  // For FP8 a negative token scale is applied exactly by negating that
  // token's codes: ReLU(s * x) = |s| * ReLU(sign(s) * x).  Whether any scale
  // of the span is negative is settled once, before the loop, so the hot
  // loop carries no branch.
  bool flip = false;
  if constexpr (!FmtInfo<FMT>::kMX) {
    if (cl < ch) {
      // 16-byte loads, 32 in flight per lane (8192 scales a round); the range
      // check zero-fills dwords past the array, and scales of columns past
      // the span only cost the exact path.
      typedef int v4i __attribute__((ext_vector_type(4)));
      constexpr int kPer = 32;
      int neg = 0;
      for (int j = cl + 4 * lane; j < ch; j += 4 * kPer * kWaveLanes) {
        v4i sv[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u)
          sv[u] = __builtin_amdgcn_raw_buffer_load_b128(sc_r, 4 * (j + 4 * kWaveLanes * u), 0, 0);
#pragma unroll
        for (int u = 0; u < kPer; ++u) neg |= (sv[u][0] | sv[u][1]) | (sv[u][2] | sv[u][3]);
      }
      flip = __ballot(neg < 0) != 0;           // any sign bit set (-0.0 is harmless)
    }
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
    __shared__ __attribute__((aligned(16))) float stage_all[kDenseWaves][2 * kRowsPerWave * kTripCols];
    float* stage = stage_all[wave];
    const int rows = min(kRowsPerWave, p.sq - row0);
    const int col4 = 4 * n;                     // lane l's group: row g, columns col4 .. col4 + 3
    const bool grp_ok = g < rows;
    const int grp_off = (int)(g * p.stride * kOB) + kOB * col4;
    const int lim = c1 & ~3;
    const float4 ninf4 = {neg_inf(), neg_inf(), neg_inf(), neg_inf()};
    // a group is stored when its row exists and it ends at or below lim
    const int last_j0 = grp_ok ? lim - col4 - 4 : -0x40000000;
    auto fill = [&](int from, int to) {          // -inf over whole trips [from, to)
      for (int j0 = from; j0 < to; j0 += kTripCols)
        OE::store4(out_r, j0 <= last_j0 ? grp_off + kOB * j0 : kOOB, ninf4);
    };
    fill(c0, cl);
    StagedSink<OUT> sink{stage, out_r, cl, g * kTripCols + n, g * kTripCols + col4, grp_off, last_j0,
                    rel_n, len, ninf4, kOOB};
    const int walked = walk(sink);
    fill(cl < ch ? walked : c1, c1);
    // The last group of a row whose Skv is not a multiple of 4: 1..3 columns,
    // one per lane, from the last trip's LDS buffer or -inf.
    if ((c1 & 3) != 0) {
      const int gs = c1 & ~3;
      if (row_ok && gs + n < c1) {
        float v = neg_inf();
        const int jt = walked - kTripCols;
        if (cl < ch && gs >= jt && gs < walked) v = sink.buffer(jt)[g * kTripCols + (gs - jt) + n];
        OE::store1(out_r, (int)(g * p.stride * kOB) + kOB * (gs + n), v);
      }
    }
  } else {
    // Keep and compressed: each in-range value goes straight to its column.
    auto off = [&](int j0, float& v) {
      (void)v;
      return (uint32_t)(j0 + rel_n) < (uint32_t)len ? lane_off + kOB * j0 : kOOB;
    };
    DwordSink<OUT, decltype(off)> sink{out_r, off, cl};
    walk(sink);
  }
}

// Row groups by chunks: block b (renumbered so each XCD gets a contiguous
// run) takes chunk b % n_chunks of 4 consecutive row groups, one per wave;
// the union of a group's ranges splits into n_chunks runs of whole trips of
// nearly equal length, so the chunks of a group do the same MFMA work.
template <int FMT, int H, int D, int STORE, int OUT, bool EXACT>
__global__ __launch_bounds__(kDenseThreads, dense_waves_per_simd(FMT, D)) void dense_kernel(DenseParams p) {
  const int lane = threadIdx.x & (kWaveLanes - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Blocks are dispatched round-robin over the 8 XCDs; renumber them so each
  // XCD gets a contiguous run of (row-group block, chunk) work and its L2
  // keeps that run's Q rows.
  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int rblock = bid / p.n_chunks;
  const int chunk = bid - rblock * p.n_chunks;
  const int row0 = (rblock * kDenseWaves + wave) * kRowsPerWave;
  if (row0 >= p.sq) return;
  auto seg = [&](int trips) {
    return GroupSeg{(int)((int64_t)chunk * trips / p.n_chunks),
                    (int)((int64_t)(chunk + 1) * trips / p.n_chunks), chunk == 0,
                    chunk == p.n_chunks - 1};
  };
  if constexpr (D == 64) dense_group32<FMT, STORE, OUT, EXACT, H>(p, row0, wave, lane, seg);
  else dense_group<FMT, H, D, STORE, OUT, EXACT>(p, row0, wave, lane, seg);
}

// Scheduled: wave w of block b is worker kDenseWaves * b + w and walks its
// piece of the work list (mqa_logits_metadata): row group g contributes
// max(trips, 1) units, one trip each (an empty group's single unit is its
// -inf fill).  Its entries schedule[worker] = (g, t) and schedule[worker + 1]
// bound the piece.  Entries are clamped, and every iteration moves to the next
// group, so any schedule contents stay in bounds and the loop ends.
template <int FMT, int H, int D, int STORE, int OUT, bool EXACT>
__global__ __launch_bounds__(kDenseThreads, 1) void dense_sched_kernel(DenseParams p) {
  const int lane = threadIdx.x & (kWaveLanes - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int worker = blockIdx.x * kDenseWaves + wave;
  if (worker >= p.num_splits) return;
  const int n_groups = (p.sq + kRowsPerWave - 1) / kRowsPerWave;
  int grp = clampi(p.sched[2 * worker], 0, n_groups);
  int t = max(p.sched[2 * worker + 1], 0);
  const int eg = clampi(p.sched[2 * worker + 2], 0, n_groups);
  const int et = max(p.sched[2 * worker + 3], 0);
  for (; grp < n_groups && (grp < eg || (grp == eg && t < et)); ++grp, t = 0) {
    const int t0 = t, g_cur = grp;
    auto seg = [&](int trips) {
      const int units = max(trips, 1);
      const int t1 = g_cur < eg ? units : min(units, et);
      return GroupSeg{t0, t1, t0 == 0, t1 >= units};
    };
    if constexpr (D == 64) dense_group32<FMT, STORE, OUT, EXACT, H>(p, grp * kRowsPerWave, wave, lane, seg);
    else dense_group<FMT, H, D, STORE, OUT, EXACT>(p, grp * kRowsPerWave, wave, lane, seg);
  }
}

template <int FMT, int H, int D, int STORE, int OUT, bool EXACT, bool SCHED>
static hipError_t launch_dense_inst(const DenseParams& p, hipStream_t stream) {
  if constexpr (SCHED) {
    const int grid = (p.num_splits + kDenseWaves - 1) / kDenseWaves;
    hipLaunchKernelGGL((dense_sched_kernel<FMT, H, D, STORE, OUT, EXACT>), dim3((unsigned)grid),
                       dim3(kDenseThreads), 0, stream, p);
  } else {
    const int rblocks = (p.sq + kRowsPerWave * kDenseWaves - 1) / (kRowsPerWave * kDenseWaves);
    const int64_t grid = (int64_t)rblocks * p.n_chunks;
    hipLaunchKernelGGL((dense_kernel<FMT, H, D, STORE, OUT, EXACT>), dim3((unsigned)grid),
                       dim3(kDenseThreads), 0, stream, p);
  }
  return hipGetLastError();
}

template <int FMT, int H, bool EXACT, int OUT, bool SCHED>
static hipError_t dispatch_store(const DenseParams& p, int d, int store, hipStream_t s) {
  if (d == 64) {
    switch (store) {
      case kDenseClean: return launch_dense_inst<FMT, H, 64, kDenseClean, OUT, EXACT, SCHED>(p, s);
      case kDenseKeep: return launch_dense_inst<FMT, H, 64, kDenseKeep, OUT, EXACT, SCHED>(p, s);
      default: return launch_dense_inst<FMT, H, 64, kCompressed, OUT, EXACT, SCHED>(p, s);
    }
  }
  switch (store) {
    case kDenseClean: return launch_dense_inst<FMT, H, 128, kDenseClean, OUT, EXACT, SCHED>(p, s);
    case kDenseKeep: return launch_dense_inst<FMT, H, 128, kDenseKeep, OUT, EXACT, SCHED>(p, s);
    default: return launch_dense_inst<FMT, H, 128, kCompressed, OUT, EXACT, SCHED>(p, s);
  }
}

// H <= 16 always runs EXACT (DenseMode, DenseMode32).
template <int FMT, int OUT, bool SCHED>
static hipError_t dispatch_h(const DenseParams& p, int h, int d, int store, bool exact,
                             hipStream_t s) {
  switch (h) {
    case 8: return dispatch_store<FMT, 8, true, OUT, SCHED>(p, d, store, s);
    case 16: return dispatch_store<FMT, 16, true, OUT, SCHED>(p, d, store, s);
    case 32:
      if (exact) return dispatch_store<FMT, 32, true, OUT, SCHED>(p, d, store, s);
      return dispatch_store<FMT, 32, false, OUT, SCHED>(p, d, store, s);
    default:
      if (exact) return dispatch_store<FMT, 64, true, OUT, SCHED>(p, d, store, s);
      return dispatch_store<FMT, 64, false, OUT, SCHED>(p, d, store, s);
  }
}

// Every (format, H, D, store mode, arithmetic) instance with logits of type
// OUT, by row chunks or (SCHED) by a work schedule.
template <int OUT, bool SCHED>
static hipError_t dispatch_fmt(int fmt, int h, int d, int store, bool exact, const DenseParams& p,
                               hipStream_t s) {
  switch (fmt) {
    case kFP8: return dispatch_h<kFP8, OUT, SCHED>(p, h, d, store, exact, s);
    case kMXFP8: return dispatch_h<kMXFP8, OUT, SCHED>(p, h, d, store, exact, s);
    default: return dispatch_h<kMXFP4, OUT, SCHED>(p, h, d, store, exact, s);
  }
}

}  // namespace mqa
