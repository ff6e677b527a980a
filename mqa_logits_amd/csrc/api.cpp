// C ABI of the weighted MQA-logits library: argument validation on the host
// (before any HIP call), kernel-configuration choice and launch on the
// caller's stream.  Declarations and contracts live in include/mqa_logits.h.
#include "mqa_logits.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <string>

#include "launch.hpp"

namespace {

thread_local std::string g_last_error;

mqa_status fail(mqa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

mqa_status ok() {
  g_last_error.clear();
  return MQA_OK;
}

mqa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(MQA_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// The kernels address each wave's output rows and the KV array through raw
// buffer resources with 32-bit offsets; every such range must stay below this
// many bytes (the kernels' out-of-range marker sits just above it).
constexpr int64_t kMaxRangeBytes = 0x7ff00000;

bool debug_enabled() {
  static const bool on = [] {
    const char* v = std::getenv("MQA_LOGITS_DEBUG");
    return v && v[0] && v[0] != '0';
  }();
  return on;
}

// Shared checks of the element formats and head shape.
mqa_status check_common(mqa_dtype dt, const void* q, const uint8_t* q_sf, const void* kv,
                        const uint8_t* kv_sf, const float* kv_scale, const void* weights,
                        mqa_float weights_type, mqa_float logits_type, int32_t h, int32_t d,
                        const char* who) {
  if (dt != MQA_FP8_E4M3 && dt != MQA_MXFP8_E4M3 && dt != MQA_MXFP4_E2M1)
    return fail(MQA_ERR_INVALID_ARG, "%s: unknown dtype %d", who, (int)dt);
  if (weights_type != MQA_F32 && weights_type != MQA_BF16)
    return fail(MQA_ERR_INVALID_ARG, "%s: unknown weights type %d", who, (int)weights_type);
  if (logits_type != MQA_F32 && logits_type != MQA_BF16)
    return fail(MQA_ERR_INVALID_ARG, "%s: unknown logits type %d", who, (int)logits_type);
  if (h != 8 && h != 16 && h != 32 && h != 64)
    return fail(MQA_ERR_UNSUPPORTED, "%s: H=%d not supported (8, 16, 32, 64)", who, h);
  if (d != 64 && d != 128)
    return fail(MQA_ERR_UNSUPPORTED, "%s: D=%d not supported (64, 128)", who, d);
  if (!q || !kv || !weights) return fail(MQA_ERR_INVALID_ARG, "%s: null q, kv or weights", who);
  if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(weights, 16))
    return fail(MQA_ERR_INVALID_ARG, "%s: q, kv and weights must be 16-byte aligned", who);
  if (dt == MQA_FP8_E4M3) {
    if (q_sf || kv_sf) return fail(MQA_ERR_INVALID_ARG, "%s: FP8 takes no block scales", who);
    if (!kv_scale) return fail(MQA_ERR_INVALID_ARG, "%s: FP8 needs kv_scale", who);
    if (!aligned(kv_scale, 4)) return fail(MQA_ERR_INVALID_ARG, "%s: kv_scale misaligned", who);
  } else {
    if (!q_sf || !kv_sf) return fail(MQA_ERR_INVALID_ARG, "%s: MX formats need q_sf and kv_sf", who);
    if (kv_scale) return fail(MQA_ERR_INVALID_ARG, "%s: MX formats take no kv_scale", who);
  }
  return MQA_OK;
}

// Chunks per row group: about as many waves as the SIMDs hold at once (a
// single dispatch round, one prologue per wave; the chunks of a row group
// carry equal work), with runs of at least one 64-token trip (few rows: more,
// shorter chunks).
int32_t pick_chunks(int32_t sq, int32_t skv, int32_t waves_per_simd) {
  const int64_t kTargetBlocks = 1024 * waves_per_simd / mqa::kDenseWaves;
  const int64_t qblocks = (sq + 4 * mqa::kDenseWaves - 1) / (4 * mqa::kDenseWaves);
  int64_t n_chunks = (kTargetBlocks + qblocks - 1) / qblocks;
  const int64_t max_chunks = (skv + 63) / 64;
  if (n_chunks > max_chunks) n_chunks = max_chunks;
  if (n_chunks < 1) n_chunks = 1;
  return (int32_t)n_chunks;
}

// The dense work schedule (mqa_logits_metadata): 4-row groups, at most
// kMaxSchedGroups of them (the metadata kernel's prefix lives in LDS), and a
// unit total that fits int32.
constexpr int64_t kMaxSchedGroups = 8192;

mqa_status check_dense_schedule(int32_t sq, int32_t skv, int32_t num_splits, const char* who) {
  if (num_splits < 1 || num_splits > 65536)
    return fail(MQA_ERR_INVALID_ARG, "%s: num_splits=%d not in [1, 65536]", who, num_splits);
  const int64_t groups = ((int64_t)sq + 3) / 4;
  if (groups > kMaxSchedGroups)
    return fail(MQA_ERR_UNSUPPORTED, "%s: a schedule covers at most %lld rows", who,
                (long long)(4 * kMaxSchedGroups));
  if (groups * (((int64_t)skv + 63) / 64 + 1) >= 0x7fffffff)
    return fail(MQA_ERR_UNSUPPORTED, "%s: Sq x Skv too large for a schedule", who);
  return MQA_OK;
}

mqa_status run_dense(mqa_dtype dt, const void* q, const uint8_t* q_sf, const void* kv,
                     const uint8_t* kv_sf, const float* kv_scale, const void* weights,
                     mqa_float weights_type, const int32_t* k_start, const int32_t* k_end,
                     const int64_t* row_off, void* out, mqa_float logits_type, int64_t stride,
                     int32_t sq, int32_t skv, int32_t h, int32_t d, int store,
                     const int32_t* schedule, int32_t num_splits, int32_t exact,
                     hipStream_t stream, const char* who) {
  if (schedule) {
    mqa_status st = check_dense_schedule(sq, skv, num_splits, who);
    if (st != MQA_OK) return st;
    if (!aligned(schedule, 4)) return fail(MQA_ERR_INVALID_ARG, "%s: schedule misaligned", who);
  }
  const int64_t row_bytes = (dt == MQA_MXFP4_E2M1 ? d / 2 : d);
  if ((int64_t)skv * row_bytes >= kMaxRangeBytes || (int64_t)skv * 16 >= kMaxRangeBytes)
    return fail(MQA_ERR_UNSUPPORTED, "%s: Skv=%d too large", who, skv);
  mqa::DenseParams p{};
  p.q = static_cast<const uint8_t*>(q);
  p.q_sf = q_sf;
  p.kv = static_cast<const uint8_t*>(kv);
  p.kv_sf = kv_sf;
  p.kv_scale = kv_scale;
  p.w = weights;
  p.k_start = k_start;
  p.k_end = k_end;
  p.row_off = row_off;
  p.out = out;
  p.stride = stride;
  p.sq = sq;
  p.skv = skv;
  p.n_chunks = pick_chunks(sq, skv, mqa::dense_waves_per_simd((int)dt, d));
  p.w_bf16 = weights_type == MQA_BF16;
  p.sched = schedule;
  p.num_splits = schedule ? num_splits : 0;
  p.exact = exact;
  const int out_type = logits_type == MQA_BF16 ? mqa::kBF16 : mqa::kF32;
  const int64_t grid =
      schedule ? ((int64_t)num_splits + mqa::kDenseWaves - 1) / mqa::kDenseWaves
               : (int64_t)((sq + 4 * mqa::kDenseWaves - 1) / (4 * mqa::kDenseWaves)) * p.n_chunks;
  if (grid > 0x7fffffff) return fail(MQA_ERR_UNSUPPORTED, "%s: problem too large", who);
  if (debug_enabled())
    fprintf(stderr,
            "[mqa_logits] %s dt=%d H=%d D=%d store=%d w=%d out=%d exact=%d Sq=%d Skv=%d chunks=%d "
            "grid=%lld\n",
            who, (int)dt, h, d, store, (int)weights_type, (int)logits_type, exact, sq, skv,
            p.n_chunks, (long long)grid);
  return hip_status(mqa::launch_dense((int)dt, h, d, store, out_type, p, stream), who);
}

mqa_status check_precision(mqa_precision precision, const char* who) {
  if (precision != MQA_PRECISION_DEFAULT && precision != MQA_PRECISION_EXACT_PRODUCTS)
    return fail(MQA_ERR_INVALID_ARG, "%s: unknown precision %d", who, (int)precision);
  return MQA_OK;
}

}  // namespace

extern "C" {

const char* mqa_last_error(void) { return g_last_error.c_str(); }

int32_t mqa_num_cus(int32_t device) {
  int n = 0;
  hipError_t e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess) {
    fail(MQA_ERR_HIP, "mqa_num_cus: %s", hipGetErrorString(e));
    return -1;
  }
  return n;
}

int32_t paged_mqa_logits_default_splits(int32_t device) {
  const int32_t n = mqa_num_cus(device);
  return n < 0 ? n : n * mqa::kWavesPerCu;
}

mqa_status mqa_logits(mqa_dtype dt, const void* q, const uint8_t* q_sf, const void* kv,
                      const uint8_t* kv_sf, const float* kv_scale, const void* weights,
                      const int32_t* k_start, const int32_t* k_end, void* logits,
                      int64_t logits_stride, int32_t sq, int32_t skv, int32_t h, int32_t d,
                      int32_t clean_logits, mqa_float weights_type, mqa_float logits_type,
                      const int32_t* schedule, int32_t num_splits, mqa_precision precision,
                      hipStream_t stream) {
  const char* who = "mqa_logits";
  if (sq < 0 || skv < 0) return fail(MQA_ERR_INVALID_ARG, "%s: negative Sq or Skv", who);
  if (logits_stride < skv) return fail(MQA_ERR_INVALID_ARG, "%s: logits_stride < Skv", who);
  mqa_status st = check_precision(precision, who);
  if (st != MQA_OK) return st;
  if (sq == 0 || skv == 0) return ok();
  st = check_common(dt, q, q_sf, kv, kv_sf, kv_scale, weights, weights_type,
                               logits_type, h, d, who);
  if (st != MQA_OK) return st;
  if (!k_start || !k_end || !logits) return fail(MQA_ERR_INVALID_ARG, "%s: null ranges or logits", who);
  if (!aligned(k_start, 4) || !aligned(k_end, 4) || !aligned(logits, 4))
    return fail(MQA_ERR_INVALID_ARG, "%s: ranges or logits misaligned", who);
  if (logits_type == MQA_BF16 && (logits_stride & 1))
    return fail(MQA_ERR_INVALID_ARG, "%s: bf16 logits need an even logits_stride", who);
  if (logits_stride * 4 * 4 >= kMaxRangeBytes)
    return fail(MQA_ERR_UNSUPPORTED, "%s: logits_stride %lld too large", who, (long long)logits_stride);
  return run_dense(dt, q, q_sf, kv, kv_sf, kv_scale, weights, weights_type, k_start, k_end,
                   nullptr, logits, logits_type, logits_stride, sq, skv, h, d,
                   clean_logits ? mqa::kDenseClean : mqa::kDenseKeep, schedule, num_splits,
                   precision == MQA_PRECISION_EXACT_PRODUCTS, stream, who);
}

mqa_status mqa_logits_compressed_offsets(const int32_t* k_start, const int32_t* k_end, int32_t sq,
                                         int32_t skv, int64_t* row_offsets, hipStream_t stream) {
  const char* who = "mqa_logits_compressed_offsets";
  if (sq < 0 || skv < 0) return fail(MQA_ERR_INVALID_ARG, "%s: negative Sq or Skv", who);
  if (!row_offsets || (sq > 0 && (!k_start || !k_end)))
    return fail(MQA_ERR_INVALID_ARG, "%s: null pointer", who);
  if (!aligned(row_offsets, 8) || !aligned(k_start, 4) || !aligned(k_end, 4))
    return fail(MQA_ERR_INVALID_ARG, "%s: misaligned pointer", who);
  return hip_status(mqa::launch_compressed_offsets(k_start, k_end, sq, skv, row_offsets, stream), who);
}

mqa_status mqa_logits_compressed(mqa_dtype dt, const void* q, const uint8_t* q_sf, const void* kv,
                                 const uint8_t* kv_sf, const float* kv_scale, const void* weights,
                                 const int32_t* k_start, const int32_t* k_end,
                                 const int64_t* row_offsets, void* logits_packed, int32_t sq,
                                 int32_t skv, int32_t h, int32_t d, mqa_float weights_type,
                                 mqa_float logits_type, const int32_t* schedule,
                                 int32_t num_splits, mqa_precision precision,
                                 hipStream_t stream) {
  const char* who = "mqa_logits_compressed";
  if (sq < 0 || skv < 0) return fail(MQA_ERR_INVALID_ARG, "%s: negative Sq or Skv", who);
  mqa_status st = check_precision(precision, who);
  if (st != MQA_OK) return st;
  if (sq == 0 || skv == 0) return ok();
  st = check_common(dt, q, q_sf, kv, kv_sf, kv_scale, weights, weights_type,
                               logits_type, h, d, who);
  if (st != MQA_OK) return st;
  if (!k_start || !k_end || !row_offsets || !logits_packed)
    return fail(MQA_ERR_INVALID_ARG, "%s: null ranges, offsets or output", who);
  if (!aligned(k_start, 4) || !aligned(k_end, 4) || !aligned(row_offsets, 8) ||
      !aligned(logits_packed, logits_type == MQA_BF16 ? 2 : 4))
    return fail(MQA_ERR_INVALID_ARG, "%s: misaligned pointer", who);
  return run_dense(dt, q, q_sf, kv, kv_sf, kv_scale, weights, weights_type, k_start, k_end,
                   row_offsets, logits_packed, logits_type, 0, sq, skv, h, d, mqa::kCompressed,
                   schedule, num_splits, precision == MQA_PRECISION_EXACT_PRODUCTS, stream, who);
}

mqa_status mqa_logits_topk(const void* logits, mqa_float logits_type, int64_t logits_stride,
                           const int32_t* k_start, const int32_t* k_end, int32_t sq,
                           int32_t skv, int32_t topk, int32_t* indices, int64_t indices_stride,
                           hipStream_t stream) {
  const char* who = "mqa_logits_topk";
  if (sq < 0 || skv < 0) return fail(MQA_ERR_INVALID_ARG, "%s: negative Sq or Skv", who);
  if (topk < 1) return fail(MQA_ERR_INVALID_ARG, "%s: topk=%d < 1", who, topk);
  if (logits_type != MQA_F32 && logits_type != MQA_BF16)
    return fail(MQA_ERR_INVALID_ARG, "%s: unknown logits type %d", who, (int)logits_type);
  if (logits_stride < skv) return fail(MQA_ERR_INVALID_ARG, "%s: logits_stride < Skv", who);
  if (indices_stride < topk) return fail(MQA_ERR_INVALID_ARG, "%s: indices_stride < topk", who);
  if ((k_start == nullptr) != (k_end == nullptr))
    return fail(MQA_ERR_INVALID_ARG, "%s: pass both k_start and k_end or neither", who);
  if (sq == 0) return ok();
  if (!indices || (skv > 0 && !logits)) return fail(MQA_ERR_INVALID_ARG, "%s: null pointer", who);
  if (!aligned(indices, 4) || !aligned(k_start, 4) || !aligned(k_end, 4) ||
      !aligned(logits, logits_type == MQA_BF16 ? 2 : 4))
    return fail(MQA_ERR_INVALID_ARG, "%s: misaligned pointer", who);
  if ((int64_t)skv * 4 >= kMaxRangeBytes)
    return fail(MQA_ERR_UNSUPPORTED, "%s: Skv=%d too large", who, skv);
  mqa::TopkParams p{logits, logits_stride, k_start, k_end, sq, skv, topk, indices,
                    indices_stride};
  return hip_status(
      mqa::launch_topk(logits_type == MQA_BF16 ? mqa::kBF16 : mqa::kF32, p, stream), who);
}

int64_t mqa_logits_metadata_size(int32_t num_splits) {
  return num_splits < 1 ? -1 : 2 * (int64_t)(num_splits + 1);
}

mqa_status mqa_logits_metadata(const int32_t* k_start, const int32_t* k_end, int32_t sq,
                               int32_t skv, int32_t num_splits, int32_t* schedule,
                               hipStream_t stream) {
  const char* who = "mqa_logits_metadata";
  if (sq < 0 || skv < 0) return fail(MQA_ERR_INVALID_ARG, "%s: negative Sq or Skv", who);
  mqa_status st = check_dense_schedule(sq, skv, num_splits, who);
  if (st != MQA_OK) return st;
  if (!schedule || (sq > 0 && (!k_start || !k_end)))
    return fail(MQA_ERR_INVALID_ARG, "%s: null pointer", who);
  if (!aligned(schedule, 4) || !aligned(k_start, 4) || !aligned(k_end, 4))
    return fail(MQA_ERR_INVALID_ARG, "%s: misaligned pointer", who);
  return hip_status(mqa::launch_dense_metadata(k_start, k_end, sq, skv, num_splits, schedule,
                                               stream),
                    who);
}

int64_t paged_mqa_logits_metadata_size(int32_t num_splits) {
  return num_splits < 1 ? -1 : 2 * (int64_t)(num_splits + 1);
}

static mqa_status check_paged_shape(int32_t batch, int32_t next_n, int32_t block_size,
                                    int32_t max_context_len, int32_t num_splits, const char* who) {
  if (batch < 1 || batch > 8192) return fail(MQA_ERR_UNSUPPORTED, "%s: batch=%d not in [1, 8192]", who, batch);
  if (next_n < 1 || next_n > 16) return fail(MQA_ERR_UNSUPPORTED, "%s: next_n=%d not in [1, 16]", who, next_n);
  if (block_size != 16 && block_size != 32 && block_size != 64)
    return fail(MQA_ERR_UNSUPPORTED, "%s: block_size=%d not in {16, 32, 64}", who, block_size);
  if (max_context_len < 0) return fail(MQA_ERR_INVALID_ARG, "%s: negative max_context_len", who);
  if (num_splits < 1 || num_splits > 65536)
    return fail(MQA_ERR_INVALID_ARG, "%s: num_splits=%d not in [1, 65536]", who, num_splits);
  const int64_t nb_max = ((int64_t)max_context_len + block_size - 1) / block_size;
  if ((int64_t)batch * nb_max >= 0x7fffffff)
    return fail(MQA_ERR_UNSUPPORTED, "%s: batch * blocks per sequence overflows int32", who);
  return MQA_OK;
}

mqa_status paged_mqa_logits_metadata(const int32_t* context_lens, int32_t batch, int32_t next_n,
                                     int32_t block_size, int32_t max_context_len, int32_t num_splits,
                                     int32_t* schedule, hipStream_t stream) {
  const char* who = "paged_mqa_logits_metadata";
  mqa_status st = check_paged_shape(batch, next_n, block_size, max_context_len, num_splits, who);
  if (st != MQA_OK) return st;
  if (!context_lens || !schedule) return fail(MQA_ERR_INVALID_ARG, "%s: null pointer", who);
  if (!aligned(context_lens, 4) || !aligned(schedule, 4))
    return fail(MQA_ERR_INVALID_ARG, "%s: misaligned pointer", who);
  return hip_status(mqa::launch_paged_metadata(context_lens, batch, block_size, max_context_len,
                                               num_splits, schedule, stream),
                    who);
}

mqa_status paged_mqa_logits(mqa_dtype dt, const void* q, const uint8_t* q_sf, const void* kv_pool,
                            const uint8_t* kv_sf_pool, const float* kv_scale_pool,
                            const void* weights, const int32_t* context_lens,
                            const int32_t* block_table, int64_t block_table_stride,
                            const int32_t* schedule, void* logits, int64_t logits_stride,
                            int32_t batch, int32_t next_n, int32_t h, int32_t d,
                            int32_t block_size, int32_t num_blocks, int32_t max_context_len,
                            int32_t num_splits, int32_t clean_logits, mqa_float weights_type,
                            mqa_float logits_type, mqa_precision precision, hipStream_t stream) {
  const char* who = "paged_mqa_logits";
  mqa_status st = check_paged_shape(batch, next_n, block_size, max_context_len, num_splits, who);
  if (st != MQA_OK) return st;
  st = check_precision(precision, who);
  if (st != MQA_OK) return st;
  st = check_common(dt, q, q_sf, kv_pool, kv_sf_pool, kv_scale_pool, weights, weights_type,
                    logits_type, h, d, who);
  if (st != MQA_OK) return st;
  if (num_blocks < 1) return fail(MQA_ERR_INVALID_ARG, "%s: num_blocks < 1", who);
  if (!context_lens || !block_table || !schedule || !logits)
    return fail(MQA_ERR_INVALID_ARG, "%s: null pointer", who);
  if (logits_stride < max_context_len)
    return fail(MQA_ERR_INVALID_ARG, "%s: logits_stride < max_context_len", who);
  const int64_t nb_max = ((int64_t)max_context_len + block_size - 1) / block_size;
  if (block_table_stride < nb_max)
    return fail(MQA_ERR_INVALID_ARG, "%s: block_table_stride < ceil(max_context_len / block_size)", who);
  if (!aligned(context_lens, 4) || !aligned(block_table, 4) || !aligned(schedule, 4) ||
      !aligned(logits, 4))
    return fail(MQA_ERR_INVALID_ARG, "%s: misaligned pointer", who);
  if (logits_type == MQA_BF16 && (logits_stride & 1))
    return fail(MQA_ERR_INVALID_ARG, "%s: bf16 logits need an even logits_stride", who);
  if ((int64_t)next_n * logits_stride * 4 >= kMaxRangeBytes)
    return fail(MQA_ERR_UNSUPPORTED, "%s: logits_stride %lld too large", who, (long long)logits_stride);
  if ((int64_t)num_blocks * block_size * 4 >= kMaxRangeBytes)
    return fail(MQA_ERR_UNSUPPORTED, "%s: pool of %d blocks too large", who, num_blocks);
  if (max_context_len == 0) return ok();
  mqa::PagedParams p{};
  p.q = static_cast<const uint8_t*>(q);
  p.q_sf = q_sf;
  p.kv = static_cast<const uint8_t*>(kv_pool);
  p.kv_sf = kv_sf_pool;
  p.kv_scale = kv_scale_pool;
  p.w = weights;
  p.ctx = context_lens;
  p.bt = block_table;
  p.bt_stride = block_table_stride;
  p.sched = schedule;
  p.out = logits;
  p.stride = logits_stride;
  p.batch = batch;
  p.next_n = next_n;
  p.bs = block_size;
  p.num_blocks = num_blocks;
  p.max_ctx = max_context_len;
  p.num_splits = num_splits;
  p.nb_max = (int32_t)nb_max;
  p.w_bf16 = weights_type == MQA_BF16;
  p.exact = precision == MQA_PRECISION_EXACT_PRODUCTS;
  if (debug_enabled())
    fprintf(stderr, "[mqa_logits] %s dt=%d H=%d D=%d batch=%d next_n=%d bs=%d splits=%d exact=%d\n",
            who, (int)dt, h, d, batch, next_n, block_size, num_splits, p.exact);
  const int out_type = logits_type == MQA_BF16 ? mqa::kBF16 : mqa::kF32;
  return hip_status(mqa::launch_paged((int)dt, h, d, clean_logits ? 1 : 0, out_type, p, stream),
                    who);
}

}  // extern "C"
