// Kernel parameter blocks and host-side launchers (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mqa {

// Output modes of the dense kernel.
enum Store : int { kDenseClean = 0, kDenseKeep = 1, kCompressed = 2 };

// Element type of the weights and of the logits (the C ABI's mqa_float).
enum FloatType : int { kF32 = 0, kBF16 = 1 };

// Waves per block of the paged kernel.  One: every value a wave needs to be
// uniform (its schedule slot, its buffer resources) then comes from blockIdx
// and the kernel arguments, which live in SGPRs already.
constexpr int kWavesPerBlock = 1;
// Waves per block of the dense kernel: one per SIMD of a compute unit, each
// on its own 4-row group, all walking the same chunk of KV columns, so a KV
// tile comes from L2 once per CU and from the CU's L1 for the other waves.
constexpr int kDenseWaves = 4;
// Resident waves per compute unit the kernels are sized for (one per SIMD).
constexpr int kWavesPerCu = 4;
// Waves per SIMD the chunked dense kernel is built for: two for e2m1 elements
// with D = 128 (their Q operands take half the registers, and a second wave's
// epilogue can run beside a 4-pass fp4 MFMA), one otherwise.  The scheduled
// kernel keeps one (its worker count is the caller's).
constexpr int dense_waves_per_simd(int fmt, int d) { return fmt == 2 && d == 128 ? 2 : 1; }
// KV operand buffers in flight per wave: a step's operands are requested
// kKvStages - 1 steps (16 tokens each) before their MFMAs issue, and a wave
// walks whole trips of kKvStages steps.
constexpr int kKvStages = 4;

struct DenseParams {
  const uint8_t* q;        // [Sq, H, D] bytes (fp4: D/2)
  const uint8_t* q_sf;     // [Sq, H, D/32] or null
  const uint8_t* kv;       // [Skv, D] bytes (fp4: D/2)
  const uint8_t* kv_sf;    // [Skv, D/32] or null
  const float* kv_scale;   // [Skv] (FP8) or null
  const void* w;           // [Sq, H] fp32 or bf16 (w_bf16)
  const int32_t* k_start;  // [Sq]
  const int32_t* k_end;    // [Sq]
  const int64_t* row_off;  // [Sq + 1] (compressed) or null
  void* out;               // fp32 or bf16 elements (the kernel's OUT)
  int64_t stride;          // dense row stride in elements
  int32_t sq, skv;
  int32_t n_chunks;        // chunks per 4-row group (each computes an equal run of the rows' range)
  int32_t w_bf16;          // weights are bf16
  const int32_t* sched;    // [num_splits + 1][2] work schedule, or null (row chunks)
  int32_t num_splits;
  int32_t exact;           // every product exact (picks the instance; see Split)
};

// Heads whose kernels split ReLU into |x| / 2 and x / 2 and take the linear
// half from the weighted query sum (RowGroup::make_lin).
constexpr int kLinHeads = 64;

struct PagedParams {
  const uint8_t* q;          // [batch*next_n, H, D]
  const uint8_t* q_sf;
  const uint8_t* kv;         // [num_blocks, bs, D]
  const uint8_t* kv_sf;      // [num_blocks, bs, D/32]
  const float* kv_scale;     // [num_blocks, bs]
  const void* w;             // [batch*next_n, H] fp32 or bf16 (w_bf16)
  const int32_t* ctx;        // [batch]
  const int32_t* bt;         // [batch, bt_stride]
  int64_t bt_stride;
  const int32_t* sched;      // [num_splits + 1][2]
  void* out;                 // fp32 or bf16 elements (the kernel's OUT)
  int64_t stride;
  int32_t batch, next_n, bs, num_blocks, max_ctx, num_splits, nb_max;
  int32_t w_bf16;
  int32_t exact;             // every product exact (picks the instance; see Split)
};

struct TopkParams {
  const void* logits;        // [Sq, stride] fp32 or bf16
  int64_t stride;            // elements
  const int32_t* k_start;    // [Sq] or null (every row is [0, Skv))
  const int32_t* k_end;      // [Sq] or null
  int32_t sq, skv, topk;
  int32_t* indices;          // [Sq, out_stride] int32
  int64_t out_stride;
};

hipError_t launch_topk(int in_type, const TopkParams& p, hipStream_t s);
hipError_t launch_dense(int fmt, int h, int d, int store, int out, const DenseParams& p,
                        hipStream_t s);
hipError_t launch_dense_f32(int fmt, int h, int d, int store, const DenseParams& p, hipStream_t s);
hipError_t launch_dense_bf16(int fmt, int h, int d, int store, const DenseParams& p, hipStream_t s);
hipError_t launch_dense_sched_f32(int fmt, int h, int d, int store, const DenseParams& p,
                                  hipStream_t s);
hipError_t launch_dense_sched_bf16(int fmt, int h, int d, int store, const DenseParams& p,
                                   hipStream_t s);
hipError_t launch_dense_metadata(const int32_t* ks, const int32_t* ke, int32_t sq, int32_t skv,
                                 int32_t num_splits, int32_t* sched, hipStream_t s);
hipError_t launch_compressed_offsets(const int32_t* ks, const int32_t* ke, int32_t sq, int32_t skv,
                                     int64_t* off, hipStream_t s);
hipError_t launch_paged(int fmt, int h, int d, int clean, int out, const PagedParams& p,
                        hipStream_t s);
hipError_t launch_paged_metadata(const int32_t* ctx, int32_t batch, int32_t bs, int32_t max_ctx,
                                 int32_t num_splits, int32_t* sched, hipStream_t s);

}  // namespace mqa
