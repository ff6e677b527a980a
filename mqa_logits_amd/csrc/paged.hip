// Paged decode weighted MQA logits and its work-split metadata for gfx950.
//
// The paged path of "How to Implement MQA (Multi-Query Attention) Logits
// Computation with DeepGEMM" (Implementing Paged MQA Logits Computation for
// Decoding): KV lives in fixed-size physical blocks reached through a block
// table, each sequence has next_n new query tokens ("[PR #314] fix: SM90
// paged MQA logits IMA on next_n=4", commit 12cb7c0), and a metadata call
// made once per decoding step splits the (sequence, KV block) work list over
// the workers (same PR, a97b74d Root cause / Fix).
//
// A worker is one block: one wave, or for clean logits with 64 heads two
// waves that split the heads (paged_kernel below).  One unit = one KV block
// for all next_n query rows of a sequence (a single query atom: producer and
// consumer of the schedule cannot disagree on atoms).  A worker holds 4 query
// rows at a time, so for next_n > 4 it walks its run of blocks once per group
// of 4 rows; the re-read blocks come from L2.  Columns past a sequence's last
// block are -inf fill units spread round-robin over the waves of the launch.
#include "common.hpp"
#include "launch.hpp"
#include "schedule.hpp"

namespace mqa {

// Clean output of a head-split worker (HS = 2 below).  Each wave stages its
// partial head sums of a trip (4 rows x kTripCols columns, -inf outside the
// rows' ranges) in its own LDS buffers; after a barrier that both waves reach
// once they have written the trip, a lane adds the two partials of one
// 4-column group and stores it: wave w stores rows 2w and 2w + 1 from lanes
// 0..31 (256-byte runs per row), lanes 32..63 store nothing.  Trips alternate
// between two buffers, so a buffer is rewritten only after the next trip's
// barrier, when both waves have read it.
template <int OUT>
struct PairSink {
  float* mine;               // this wave's 2 x [4][kTripCols] floats
  const float* other;        // the partner wave's
  Rsrc r;
  int base;                  // first column of the walk (trip-aligned)
  int put_idx;               // this lane's slot: row g, column n of a trip's first step
  int rd_idx;                // this lane's store group in a buffer
  int row_off;               // byte offset of that group in the output at column 0
  int last_j0;               // the group of trip j0 is stored iff base <= j0 <= last_j0
  int rel_n, len;            // column j0 + n is in range iff j0 + rel_n in [0, len)
  float4 pend;               // the last trip's sums, and their store offset
  int pend_off;

  __device__ __forceinline__ int half(int j0) const {
    return (((j0 - base) >> 6) & 1) * (kRowsPerWave * kTripCols);
  }
  __device__ __forceinline__ void put(int u, int j0, float v) {
    const bool in_range = (uint32_t)(j0 + rel_n) < (uint32_t)len;
    mine[half(j0) + put_idx + u * kTileN] = in_range ? v : neg_inf();
    if (u == 0) OutElem<OUT>::store4(r, pend_off, pend);
  }
  __device__ __forceinline__ void trip(int jt) {
    // both waves' writes of trip jt are done (LDS only: the KV loads in
    // flight are not waited for)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const float4 a = *reinterpret_cast<const float4*>(mine + half(jt) + rd_idx);
    const float4 b = *reinterpret_cast<const float4*>(other + half(jt) + rd_idx);
    pend = float4{a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w};
    pend_off = (jt <= last_j0 ? row_off + OutElem<OUT>::kBytes * jt : kOOB) | oob_if(jt < base);
    asm volatile("" ::: "memory");
  }
  __device__ __forceinline__ void finish() { OutElem<OUT>::store4(r, pend_off, pend); }
};

// HS = 1: one wave per worker holds all H heads.  HS = 2 (clean output,
// H = 64): the two waves of a block split the heads of one worker -- each
// holds H / 2 heads' Q operands and weights, about half the registers, so two
// workers share a SIMD and one's gather latency hides behind the other's
// math -- walk the same blocks (the second read of a KV step comes from the
// cache) and add their partial sums in PairSink.  Both waves take identical,
// wave-uniform control flow, so they meet every barrier.
//
// EXACT: every product reaches the accumulator exactly (Split; always for
// H <= 16, on request otherwise).
template <int FMT, int H, int D, bool CLEAN, int OUT, int HS, bool EXACT>
__global__ __launch_bounds__(kWaveLanes * HS, HS) void paged_kernel(PagedParams p) {
  static_assert(HS == 1 || (HS == 2 && CLEAN), "the head split writes clean logits only");
  // The linear half of ReLU on the matrix core was measured not to pay off
  // for decode batches, so the paged kernel keeps max + fma.
  using RG = RowGroup<FMT, H / HS, D, false, EXACT || H <= 16>;
  using L = OperandLayout<FMT, D>;
  using OE = OutElem<OUT>;
  constexpr int kOB = OE::kBytes;              // bytes per logits element
  constexpr int kNKB = RG::kNKB;
  constexpr int kRowBytes = RG::kRowBytes;
  constexpr int kBtWindow = kWaveLanes;        // block-table entries held per lane

  const int lane = threadIdx.x & (kWaveLanes - 1);
  const int wave = HS == 1 ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int worker = blockIdx.x;                // HS waves per block
  if (worker >= p.num_splits) return;

  const int g = lane >> 4;                 // output row (query token) of this lane in its group
  const int n = lane & 15;                 // column within a 16-token tile
  const int kb = lane >> 4;                // lane group: operand pieces and scale block
  const bool kb_ok = L::scale_ok(kb);
  const int n_groups = (p.next_n + kRowsPerWave - 1) / kRowsPerWave;
  const int bs = p.bs;
  const int bs_shift = 31 - __builtin_clz(bs);

  // operand lanes: token n of the step, the lane group's two 16-byte pieces
  const int b_lo = L::lo(kb) >= 0 ? n * kRowBytes + L::lo(kb) : kOOB;
  const int b_hi = L::hi(kb) >= 0 ? n * kRowBytes + L::hi(kb) : kOOB;
  const int64_t pool_tokens = (int64_t)p.num_blocks * bs;
  Rsrc sc_r;
  if constexpr (FmtInfo<FMT>::kMX) {
    sc_r = make_rsrc(p.kv_sf, (uint32_t)(pool_tokens * kNKB));
  } else {
    sc_r = make_rsrc(p.kv_scale, (uint32_t)(pool_tokens * 4));
  }

  int b = max(p.sched[2 * worker], 0);
  int blk = max(p.sched[2 * worker + 1], 0);
  const int eb = p.sched[2 * worker + 2];
  const int eblk = p.sched[2 * worker + 3];

  __shared__ __attribute__((aligned(16))) float stage_all[HS][2 * kRowsPerWave * kTripCols];
  float* const stage = stage_all[wave];
  const float4 ninf4 = {neg_inf(), neg_inf(), neg_inf(), neg_inf()};
  if constexpr (CLEAN) {
    // -inf for the blocks past each sequence's last one, round-robin over
    // the waves of the launch: this wave owns units me, me + P, ...  Lane l
    // looks up unit me + (64 k + l) P, so one load serves 64 units and no
    // store waits on a load issued after it.  The fill goes first: at the
    // wave's end it would add a store round trip to the launch's tail; here
    // its stores drain while the first operands of the walk are loading.
    const int64_t total = (int64_t)p.batch * p.nb_max;
    const int64_t P = (int64_t)p.num_splits * HS;
    for (int64_t f0 = worker + (int64_t)wave * p.num_splits; f0 < total; f0 += P * kWaveLanes) {
      const int64_t f = f0 + (int64_t)lane * P;
      int fb = 0, c = 0;
      bool need = false;
      if (f < total) {
        fb = (int)(f / p.nb_max);
        c = (int)(f - (int64_t)fb * p.nb_max);
        const int len = clampi(p.ctx[fb], 0, p.max_ctx);
        need = c >= ((len + bs - 1) >> bs_shift);
      }
      for (uint64_t m = __ballot(need); m != 0; m &= m - 1) {
        const int k = __builtin_ctzll(m);
        const int ub = __builtin_amdgcn_readlane(fb, k);
        const int uc = __builtin_amdgcn_readlane(c, k);
        const Rsrc out_r = make_rsrc(static_cast<char*>(p.out) + (int64_t)ub * p.next_n * p.stride * kOB,
                                     (uint32_t)(p.next_n * p.stride * kOB));
        // 16-byte groups (lane l: row l / 16 of a 4-row group, columns
        // 4 (l % 16) .. +3), then the 1..3 columns of a last group cut by max_ctx
        const int c0 = uc << bs_shift;
        const int c1 = min((uc + 1) << bs_shift, p.max_ctx);
        for (int t0 = 0; t0 < p.next_n; t0 += kRowsPerWave) {
          const bool row_ok = t0 + g < p.next_n;
          const int t_e = min(t0 + g, p.next_n - 1);
          const int grp_off = (t_e * (int)p.stride + 4 * n) * kOB;
          for (int j0 = c0; j0 < c1; j0 += kTripCols)
            OE::store4(out_r, (row_ok && j0 + 4 * n + 4 <= c1) ? grp_off + kOB * j0 : kOOB, ninf4);
          if ((c1 & 3) != 0 && row_ok && (c1 & ~3) + n < c1 && (c1 & ~3) >= c0)
            OE::store1(out_r, (t_e * (int)p.stride + (c1 & ~3) + n) * kOB, neg_inf());
        }
      }
    }
  }
  RG rg;
  while (b < p.batch && (b < eb || (b == eb && blk < eblk))) {
    const int ctx = p.ctx[b];
    const int len = clampi(ctx, 0, p.max_ctx);
    const int n_b = (len + bs - 1) >> bs_shift;
    if (blk >= n_b) {                      // past this sequence: next one
      ++b;
      blk = 0;
      continue;
    }
    // this worker's blocks of sequence b: [blk, seg_end)
    const int seg_end = b < eb ? n_b : min(n_b, eblk);
    const int64_t r0 = (int64_t)b * p.next_n;
    for (int grp = 0; grp < n_groups; ++grp) {
      const int t0 = grp * kRowsPerWave;
      const bool row_ok = t0 + g < p.next_n;
      const int t_e = min(t0 + g, p.next_n - 1);
      const int t_a = min(t0 + ((lane >> 2) & 3), p.next_n - 1);
      rg.load(p.q, p.q_sf, p.w, p.w_bf16 != 0, r0 + t_a, r0 + t_e, lane, H, wave * (H / HS));
      const int e_tok = clampi(ctx - p.next_n + t_e + 1, 0, len);   // this lane's row end
      const Rsrc out_r = make_rsrc(static_cast<char*>(p.out) + r0 * p.stride * kOB,
                                   (uint32_t)(p.next_n * p.stride * kOB));
      const int lane_off = (t_e * (int)p.stride + n) * kOB;
      const int rel_n = n - e_tok;           // j0 + rel_n < 0  iff  column in range

      for (int sub = blk; sub < seg_end; sub += kBtWindow) {
        const int cnt = min(kBtWindow, seg_end - sub);
        const int bt_lane = clampi(p.bt[(int64_t)b * p.bt_stride + sub + min(lane, cnt - 1)], 0,
                                   p.num_blocks - 1);
        const int col0 = sub << bs_shift;
        const int col1 = min((sub + cnt) << bs_shift, p.max_ctx);
        const int wlim_n = (row_ok ? col1 : 0) - n;

        auto load = [&](int j0, KvOp& o) {
          const int bi = min((j0 >> bs_shift) - sub, cnt - 1);
          const int pblk = __builtin_amdgcn_readlane(bt_lane, bi);
          const int tok = (pblk << bs_shift) + (j0 & (bs - 1));   // first pool token of the step
          const Rsrc kv_r = make_rsrc(p.kv + (int64_t)tok * kRowBytes, kTileN * kRowBytes);
          o.b = buffer_operand(kv_r, b_lo, b_hi);
          if constexpr (FmtInfo<FMT>::kMX) {
            // lanes past the row's scale blocks (D = 64) read 0 past the
            // buffer's end: their operand pieces are zero, so any finite
            // scale serves, and the load needs no branch
            o.bs = __builtin_amdgcn_raw_buffer_load_b8(sc_r, kb_ok ? (tok + n) * kNKB + kb : kOOB, 0, 0);
            o.ks = 1.f;
          } else {
            o.bs = 127;
            o.ks = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(sc_r, (tok + n) * 4, 0, 0));
          }
        };
        // Paged decode is bound by the KV gather, so FP8 always takes the
        // sign-exact path (negative token scales negate the token's codes)
        // instead of scanning the scales first.
        constexpr bool kFlip = !FmtInfo<FMT>::kMX;
        KvOp o[kKvStages];
        prefetch_span(col0, o, load);
        if constexpr (CLEAN && HS == 2) {
          const int rs = 2 * wave + ((lane >> 4) & 1);   // the row this lane stores
          const bool st_ok = lane < 32 && t0 + rs < p.next_n;
          const int t_s = min(t0 + rs, p.next_n - 1);
          const int last_j0 = st_ok ? (col1 & ~3) - 4 * n - 4 : -0x40000000;
          PairSink<OUT> sink{stage,     stage_all[wave ^ 1], out_r,  col0,
                             g * kTripCols + n, rs * kTripCols + 4 * n,
                             (t_s * (int)p.stride + 4 * n) * kOB, last_j0, n, e_tok, ninf4, kOOB};
          const int walked = compute_span<kFlip>(rg, col0, col1, o, load, sink);
          if ((col1 & 3) != 0) {             // max_ctx not a multiple of 4: 1..3 columns
            const int gs = col1 & ~3, jt = walked - kTripCols;
            if (wave == 0 && row_ok && gs + n < col1) {
              float v = neg_inf();
              if (gs >= jt && gs < walked) {
                const int i = sink.half(jt) + g * kTripCols + (gs - jt) + n;
                v = stage_all[0][i] + stage_all[1][i];
              }
              OE::store1(out_r, (t_e * (int)p.stride + gs + n) * kOB, v);
            }
          }
          // the partner's next walk rewrites its buffers only after this
          // wave's last reads of them
          asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        } else if constexpr (CLEAN) {
          // Whole 16-byte groups of the window through LDS (lane l: row l / 16,
          // columns 4 (l % 16) .. +3 of a trip); in range iff column < e_tok.
          const int lim = col1 & ~3;
          const int last_j0 = row_ok ? lim - 4 * n - 4 : -0x40000000;
          StagedSink<OUT> sink{stage, out_r, col0, g * kTripCols + n, g * kTripCols + 4 * n,
                               (t_e * (int)p.stride + 4 * n) * kOB, last_j0, n, e_tok, ninf4, kOOB};
          const int walked = compute_span<kFlip>(rg, col0, col1, o, load, sink);
          if ((col1 & 3) != 0) {             // max_ctx not a multiple of 4: 1..3 columns
            const int gs = col1 & ~3, jt = walked - kTripCols;
            if (row_ok && gs + n < col1) {
              float v = neg_inf();
              if (gs >= jt && gs < walked) v = sink.buffer(jt)[g * kTripCols + (gs - jt) + n];
              OE::store1(out_r, (t_e * (int)p.stride + gs + n) * kOB, v);
            }
          }
        } else {
          auto off = [&](int j0, float& v) {
            (void)v;
            return (j0 < wlim_n && j0 + rel_n < 0) ? lane_off + kOB * j0 : kOOB;
          };
          DwordSink<OUT, decltype(off)> sink{out_r, off, col0};
          compute_span<kFlip>(rg, col0, col1, o, load, sink);
        }
      }
    }
    blk = seg_end;
  }
}

// One block per worker: clean logits with 64 heads split the heads over two
// waves (not EXACT: its eight KV operand copies want the registers the split
// saves), everything else runs one wave per worker.
template <int FMT, int H, int D, int OUT, bool EXACT>
static hipError_t launch_paged_inst(int clean, const PagedParams& p, hipStream_t s) {
  const int grid = p.num_splits;
  if (clean) {
    constexpr int kHS = (H == 64 && !EXACT) ? 2 : 1;
    hipLaunchKernelGGL((paged_kernel<FMT, H, D, true, OUT, kHS, EXACT>), dim3(grid),
                       dim3(kWaveLanes * kHS), 0, s, p);
  } else {
    hipLaunchKernelGGL((paged_kernel<FMT, H, D, false, OUT, 1, EXACT>), dim3(grid),
                       dim3(kWaveLanes), 0, s, p);
  }
  return hipGetLastError();
}

template <int FMT, int H, int OUT, bool EXACT>
static hipError_t paged_d(int d, int clean, const PagedParams& p, hipStream_t s) {
  return d == 64 ? launch_paged_inst<FMT, H, 64, OUT, EXACT>(clean, p, s)
                 : launch_paged_inst<FMT, H, 128, OUT, EXACT>(clean, p, s);
}

// H <= 16 always runs exact; MXFP4 products are exact without the split.
template <int FMT, int OUT>
static hipError_t paged_h(int h, int d, int clean, const PagedParams& p, hipStream_t s) {
  const bool exact = p.exact != 0 && FMT != kMXFP4;
  switch (h) {
    case 8: return paged_d<FMT, 8, OUT, true>(d, clean, p, s);
    case 16: return paged_d<FMT, 16, OUT, true>(d, clean, p, s);
    case 32:
      return exact ? paged_d<FMT, 32, OUT, true>(d, clean, p, s)
                   : paged_d<FMT, 32, OUT, false>(d, clean, p, s);
    default:
      return exact ? paged_d<FMT, 64, OUT, true>(d, clean, p, s)
                   : paged_d<FMT, 64, OUT, false>(d, clean, p, s);
  }
}

template <int OUT>
static hipError_t paged_fmt(int fmt, int h, int d, int clean, const PagedParams& p, hipStream_t s) {
  switch (fmt) {
    case kFP8: return paged_h<kFP8, OUT>(h, d, clean, p, s);
    case kMXFP8: return paged_h<kMXFP8, OUT>(h, d, clean, p, s);
    default: return paged_h<kMXFP4, OUT>(h, d, clean, p, s);
  }
}

hipError_t launch_paged(int fmt, int h, int d, int clean, int out, const PagedParams& p,
                        hipStream_t s) {
  return out == kBF16 ? paged_fmt<kBF16>(fmt, h, d, clean, p, s)
                      : paged_fmt<kF32>(fmt, h, d, clean, p, s);
}

// ---------------------------------------------------------------------------
// Metadata: sequence b has ceil(min(ctx_b, max_ctx) / bs) units.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kMetaThreads) void paged_metadata_kernel(
    const int32_t* __restrict__ ctx, int32_t batch, int32_t bs, int32_t max_ctx,
    int32_t num_splits, int32_t* __restrict__ sched) {
  split_units(batch, num_splits, sched, [&](int b) {
    const int len = clampi(ctx[b], 0, max_ctx);
    return (len + bs - 1) / bs;
  });
}

hipError_t launch_paged_metadata(const int32_t* ctx, int32_t batch, int32_t bs, int32_t max_ctx,
                                 int32_t num_splits, int32_t* sched, hipStream_t s) {
  hipLaunchKernelGGL(paged_metadata_kernel, dim3(1), dim3(kMetaThreads), 0, s, ctx, batch, bs,
                     max_ctx, num_splits, sched);
  return hipGetLastError();
}

}  // namespace mqa
