// Dense and compressed weighted MQA logits for gfx950.
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
// Work split: a block is one wave; it owns 4 consecutive query rows and one
// chunk of KV columns, keeps the rows' Q operands and weights in registers
// and walks the chunk 16 tokens at a time.  Tokens outside the
// union of its rows' ranges are -inf fill (no MFMA); tokens inside are
// computed and masked per row in the same store.  No second pass, no atomics:
// each output element is written by exactly one lane.
#include "common.hpp"
#include "launch.hpp"

namespace mqa {

template <int FMT, int H, int D, int STORE>
__global__ __launch_bounds__(kThreads, 1) void dense_kernel(DenseParams p) {
  using RG = RowGroup<FMT, H, D>;
  using L = OperandLayout<FMT, D>;
  constexpr int kNKB = RG::kNKB;
  constexpr int kRowBytes = RG::kRowBytes;

  const int lane = threadIdx.x & (kWaveLanes - 1);

  // Blocks (one wave each) are dispatched round-robin over the 8 XCDs;
  // renumber them so each XCD gets a contiguous run of (row group, chunk)
  // work and its L2 keeps that run's Q rows.
  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int rgroup = bid / p.n_chunks;
  const int chunk = bid - rgroup * p.n_chunks;

  const int row0 = rgroup * kRowsPerWave;
  if (row0 >= p.sq) return;

  // ---- this wave's 4 rows ----------------------------------------------
  const int g = lane >> 4;                     // output row of this lane
  const int n = lane & 15;                     // output column in a 16-token tile
  const int e_row = row0 + g;
  const bool row_ok = e_row < p.sq;
  const int e_row_c = min(e_row, p.sq - 1);
  const int a_row_c = min(row0 + ((lane >> 2) & 3), p.sq - 1);

  RG rg;
  rg.load(p.q, p.q_sf, p.w, a_row_c, e_row_c, lane);

  const int s_row = clampi(p.k_start[e_row_c], 0, p.skv);
  int e_end = clampi(p.k_end[e_row_c], s_row, p.skv);
  if (!row_ok) e_end = s_row;
  // stores stay inside this block's chunk [c0, c1) (set below)
  int len;

  // Union of the 4 rows' ranges (wave-uniform).
  int lo = 0x7fffffff, hi = 0;
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) {
    const int s_r = __builtin_amdgcn_readlane(s_row, 16 * r);
    const int e_r = __builtin_amdgcn_readlane(e_end, 16 * r);
    if (e_r > s_r) {
      lo = min(lo, s_r);
      hi = max(hi, e_r);
    }
  }

  const int c0 = chunk * p.chunk_cols;
  const int c1 = min(c0 + p.chunk_cols, p.skv);
  int cl = max(c0, lo & ~(kTileN - 1));
  int ch = min(c1, hi);
  if (cl >= ch) { cl = c1; ch = c1; }          // nothing to compute in this chunk
  len = max(0, min(e_end, c1) - s_row);

  // ---- output addressing: one buffer resource per wave -------------------
  // byte offset of (this lane's row, column 0) inside the wave's region
  Rsrc out_r;
  int lane_off;
  if constexpr (STORE == kCompressed) {
    const int64_t first = p.row_off[row0];
    const int64_t last = p.row_off[min(row0 + kRowsPerWave, p.sq)];
    out_r = make_rsrc(p.out + first, (uint32_t)((last - first) * 4));
    lane_off = (int)(row_ok ? (p.row_off[e_row_c] - first - s_row) * 4 : 0);
  } else {
    const int rows = min(kRowsPerWave, p.sq - row0);
    out_r = make_rsrc(p.out + (int64_t)row0 * p.stride, (uint32_t)(rows * p.stride * 4));
    lane_off = (int)(g * p.stride * 4);
  }
  lane_off += 4 * n;
  // clean stores write columns [c0, c1) of valid rows, in-range or -inf
  const int wlim_n = (row_ok ? c1 : 0) - n;    // column j0 + n is writable iff j0 < wlim_n
  const int rel_n = n - s_row;                 // (j0 + rel_n) in [0, len) iff in range

  // ---- -inf fill of whole tiles left of the computed span ----------------
  if constexpr (STORE == kDenseClean) {
    for (int j0 = c0; j0 < cl; j0 += kTileN)
      buffer_store_nt(out_r, j0 < wlim_n ? lane_off + 4 * j0 : kOOB, neg_inf());
  }

  // ---- computed tiles ------------------------------------------------------
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
    o.b = buffer_operand(kv_r, b_lo == kOOB ? kOOB : b_lo + j0 * kRowBytes,
                         b_hi == kOOB ? kOOB : b_hi + j0 * kRowBytes);
    if constexpr (FmtInfo<FMT>::kMX) {
      o.bs = kb_ok ? (int)__builtin_amdgcn_raw_buffer_load_b8(sc_r, sc_lane + j0 * kNKB, 0, 0) : 127;
      o.ks = 1.f;
    } else {
      o.bs = 127;
      o.ks = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(sc_r, sc_lane + 4 * j0, 0, 0));
    }
  };

  // For FP8 a negative token scale is applied exactly by negating that
  // token's codes: ReLU(s * x) = |s| * ReLU(sign(s) * x).  Whether any scale
  // of the span is negative is settled once, before the loop, so the hot
  // loop carries no branch.
  bool flip = false;
  if constexpr (!FmtInfo<FMT>::kMX) {
    if (cl < ch) {
      // dword loads: each is wholly inside or outside the scale array
      int neg = 0;
      for (int j = cl + lane; j < ch; j += 16 * kWaveLanes) {
        int s16[16];
#pragma unroll
        for (int u = 0; u < 16; ++u)
          s16[u] = __builtin_amdgcn_raw_buffer_load_b32(sc_r, 4 * (j + kWaveLanes * u), 0, 0);
#pragma unroll
        for (int u = 0; u < 16; ++u) neg |= s16[u];
      }
      flip = __ballot(neg < 0) != 0;           // any sign bit set (-0.0 is harmless)
    }
  }

  int walked = ch;
  if (cl < ch) {
    if (flip) {
      walked = compute_span<true>(rg, cl, ch, load_b, [&](int j0, float v) {
        const bool in_range = (uint32_t)(j0 + rel_n) < (uint32_t)len;
        if constexpr (STORE == kDenseClean) {
          buffer_store_nt(out_r, j0 < wlim_n ? lane_off + 4 * j0 : kOOB, in_range ? v : neg_inf());
        } else {
          buffer_store_nt(out_r, in_range ? lane_off + 4 * j0 : kOOB, v);
        }
      });
    } else {
      walked = compute_span<false>(rg, cl, ch, load_b, [&](int j0, float v) {
        const bool in_range = (uint32_t)(j0 + rel_n) < (uint32_t)len;
        if constexpr (STORE == kDenseClean) {
          buffer_store_nt(out_r, j0 < wlim_n ? lane_off + 4 * j0 : kOOB, in_range ? v : neg_inf());
        } else {
          buffer_store_nt(out_r, in_range ? lane_off + 4 * j0 : kOOB, v);
        }
      });
    }
  }

  // ---- -inf fill of whole tiles right of the computed span ---------------
  if constexpr (STORE == kDenseClean) {
    const int start = cl < ch ? walked : c1;
    for (int j0 = start; j0 < c1; j0 += kTileN)
      buffer_store_nt(out_r, j0 < wlim_n ? lane_off + 4 * j0 : kOOB, neg_inf());
  }
}

template <int FMT, int H, int D, int STORE>
static hipError_t launch_dense_inst(const DenseParams& p, hipStream_t stream) {
  const int rgroups = (p.sq + kRowsPerWave - 1) / kRowsPerWave;
  const int64_t grid = (int64_t)rgroups * p.n_chunks;
  hipLaunchKernelGGL((dense_kernel<FMT, H, D, STORE>), dim3((unsigned)grid), dim3(kThreads), 0,
                     stream, p);
  return hipGetLastError();
}

template <int FMT, int H, int D>
static hipError_t dispatch_store(const DenseParams& p, int store, hipStream_t s) {
  switch (store) {
    case kDenseClean: return launch_dense_inst<FMT, H, D, kDenseClean>(p, s);
    case kDenseKeep: return launch_dense_inst<FMT, H, D, kDenseKeep>(p, s);
    default: return launch_dense_inst<FMT, H, D, kCompressed>(p, s);
  }
}

template <int FMT, int H>
static hipError_t dispatch_d(const DenseParams& p, int d, int store, hipStream_t s) {
  return d == 64 ? dispatch_store<FMT, H, 64>(p, store, s) : dispatch_store<FMT, H, 128>(p, store, s);
}

template <int FMT>
static hipError_t dispatch_h(const DenseParams& p, int h, int d, int store, hipStream_t s) {
  switch (h) {
    case 8: return dispatch_d<FMT, 8>(p, d, store, s);
    case 16: return dispatch_d<FMT, 16>(p, d, store, s);
    case 32: return dispatch_d<FMT, 32>(p, d, store, s);
    default: return dispatch_d<FMT, 64>(p, d, store, s);
  }
}

hipError_t launch_dense(int fmt, int h, int d, int store, const DenseParams& p, hipStream_t s) {
  switch (fmt) {
    case kFP8: return dispatch_h<kFP8>(p, h, d, store, s);
    case kMXFP8: return dispatch_h<kMXFP8>(p, h, d, store, s);
    default: return dispatch_h<kMXFP4>(p, h, d, store, s);
  }
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
