/*
 * mqa_logits.h -- C ABI of the MI355X (gfx950) weighted MQA-logits library.
 *
 * The operation ("Math Warp Reduction" and "Compressed Logits" in
 * "How to Implement MQA (Multi-Query Attention) Logits Computation with
 * DeepGEMM", section Core Architecture Components; clean -inf output as in
 * "[PR #435] Improve SM100 MX MQA logits clean-output performance",
 * Description and reproducer):
 *
 *   logits[i, j] = sum_h w[i, h] * ReLU(kv_scale[j] * <q[i, h, :], kv[j, :]>)
 *                  for s_i <= j < e_i,
 *   logits[i, j] = -inf elsewhere (clean logits),
 *
 * with one KV head shared by all H query heads.  The range of row i is
 * s_i = clamp(k_start[i], 0, Skv), e_i = clamp(k_end[i], s_i, Skv); a row with
 * k_end <= k_start is empty.  For MX formats the per-token kv_scale is 1 and
 * every group of 32 consecutive elements along D carries an e8m0 scale
 * 2^(byte - 127) that multiplies those elements.
 *
 * Conventions shared by every entry point:
 *   - Every pointer argument is DEVICE memory owned by the caller.  The
 *     library allocates no device memory, keeps no state between calls and
 *     never waits for the device: all work is enqueued on `stream` (0 = the
 *     null stream), so every call may be captured into a HIP graph.
 *   - Layouts are dense row-major, strides in elements unless stated.
 *   - q, kv, kv_pool: fp8 e4m3fn bytes ([.., D]) or, for MXFP4, packed e2m1
 *     bytes ([.., D/2], element 2k in the low nibble of byte k).
 *   - q_sf, kv_sf: e8m0 bytes [.., D/32]; byte b of a row scales elements
 *     [32b, 32b+32).  (Four scale bytes of a D = 128 row are the little-endian
 *     bytes of the int32 the pages pass.)  Must be NULL for MQA_FP8_E4M3.
 *   - Pointers must be 16-byte aligned; D must be 64 or 128; H must be 8, 16,
 *     32 or 64.
 *   - Errors found on the host (NULL or misaligned pointers, sizes out of
 *     range, an unsupported H/D/format, strides below the row width) return
 *     MQA_ERR_INVALID_ARG or MQA_ERR_UNSUPPORTED before any HIP call.  A HIP
 *     error returns MQA_ERR_HIP.  mqa_last_error() then describes it.
 *   - Contents of device arrays (ranges, lengths, block ids, offsets) are
 *     preconditions the host cannot see.  Ranges are clamped on the device as
 *     above, so any int32 range is safe; block ids must lie in
 *     [0, num_blocks) and row_offsets must be the ones
 *     mqa_logits_compressed_offsets writes.
 */
#ifndef MQA_LOGITS_H
#define MQA_LOGITS_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MQA_OK = 0,
  MQA_ERR_INVALID_ARG = 1,
  MQA_ERR_UNSUPPORTED = 2,
  MQA_ERR_HIP = 3
} mqa_status;

typedef enum {
  MQA_FP8_E4M3 = 0,    /* e4m3fn Q and KV, fp32 per-token kv_scale          */
  MQA_MXFP8_E4M3 = 1,  /* e4m3fn elements + e8m0 scale per 32, no kv_scale  */
  MQA_MXFP4_E2M1 = 2   /* packed e2m1 elements + e8m0 scale per 32          */
} mqa_dtype;

/*
 * Element type of the weights and of the logits ("[PR #435] Improve SM100 MX
 * MQA logits clean-output performance", Validation: FP32 and BF16 weights and
 * output; the logits_dtype argument of its reproducer).  The arithmetic is
 * fp32 either way: bf16 weights are widened exactly, and bf16 logits are the
 * fp32 results rounded to nearest (ties to even); -inf stays -inf.
 */
typedef enum {
  MQA_F32 = 0,
  MQA_BF16 = 1
} mqa_float;

/*
 * Arithmetic of the contraction <q[i,h,:], kv[j,:]> (the pages fix only fp8
 * inputs and fp32 outputs; "How to Implement MQA (Multi-Query Attention)
 * Logits Computation with DeepGEMM", Core Architecture Components, runs the
 * product on the tensor cores).
 *
 * MQA_PRECISION_DEFAULT: the matrix core's own summation.  For FP8 and MXFP8
 *   elements with H = 32 or 64, each aligned group of 8 consecutive products
 *   along D is summed after every product is truncated toward zero to a
 *   multiple of 2^(E - 13), E = floor(log2) of the group's largest |product|
 *   (block scales included); group sums add in fp32.  A dot's error is then
 *   below sum over groups of 7 * 2^(E - 13) <= 2^-10.2 * sum_d |q_d kv_d|: it
 *   is bounded by the products, not by the dot, so cancelling dots can lose
 *   all their low bits.  With H = 64, and with H = 32 when D = 64, the
 *   linear half of ReLU comes from the weighted query sum rounded to four
 *   e4m3 pieces (about 2^-16 of each 32-element block's largest magnitude),
 *   in every format.  Products are exact in this mode too for H <= 16 and
 *   for MXFP4 elements (as below).  Block scales spread over many octaves
 *   reach the same error class as cancelling dots: a dot is then dominated
 *   by its largest-scaled blocks.
 * MQA_PRECISION_EXACT_PRODUCTS: every product reaches the fp32 accumulation
 *   exactly (the KV operand is issued once per element of each group of 8),
 *   and ReLU is evaluated per head.  For FP8 and MXFP8 with H = 32 or 64 this
 *   costs eight times the matrix-core work of the default.
 */
typedef enum {
  MQA_PRECISION_DEFAULT = 0,
  MQA_PRECISION_EXACT_PRODUCTS = 1
} mqa_precision;

/*
 * Dense logits ("Implementing Standard MQA Logits Computation" in the DeepGEMM
 * MQA-logits article; the clean_logits flag of the reproducer in PR #435).
 *   q        [Sq, H, D] (fp4: [Sq, H, D/2])      q_sf  [Sq, H, D/32] or NULL
 *   kv       [Skv, D]   (fp4: [Skv, D/2])        kv_sf [Skv, D/32]  or NULL
 *   kv_scale [Skv] fp32 for MQA_FP8_E4M3, NULL for MX formats
 *   weights  [Sq, H] of weights_type;  k_start, k_end [Sq] int32
 *   logits   [Sq, logits_stride] of logits_type, logits_stride >= Skv (even
 *            for bf16; the pointer 4-byte aligned).  Columns
 *            [Skv, logits_stride) are never written.
 *   clean_logits != 0: entries outside a row's range are written as -inf;
 *   clean_logits == 0: they are left untouched.
 *   schedule, num_splits: NULL (the rows' work is split into equal column
 *            chunks), or a work schedule from mqa_logits_metadata for these
 *            k_start, k_end, Sq, Skv and num_splits; the output is bit for bit
 *            the same either way.
 *   precision: mqa_precision above.
 * Sq == 0 or Skv == 0 is a no-op that returns MQA_OK.
 */
mqa_status mqa_logits(mqa_dtype dt,
                      const void* q, const uint8_t* q_sf,
                      const void* kv, const uint8_t* kv_sf,
                      const float* kv_scale, const void* weights,
                      const int32_t* k_start, const int32_t* k_end,
                      void* logits, int64_t logits_stride,
                      int32_t sq, int32_t skv, int32_t h, int32_t d,
                      int32_t clean_logits, mqa_float weights_type, mqa_float logits_type,
                      const int32_t* schedule, int32_t num_splits, mqa_precision precision,
                      hipStream_t stream);

/*
 * Work schedule for mqa_logits / mqa_logits_compressed (the schedule_meta of
 * the reproducer in "[PR #435] Improve SM100 MX MQA logits clean-output
 * performance", made by get_mqa_logits_metadata from the ranges; Validation
 * requires the scheduled output to equal the unscheduled one).
 *
 * Work units: rows are taken in groups of 4 (group g = rows 4g .. 4g+3).  With
 * s_i, e_i the clamped ranges, a group whose rows are all empty has one unit;
 * otherwise, with lo = min s_i and hi = max e_i over its non-empty rows, it has
 * ceil((hi - (lo & ~63)) / 64) units (64-column trips of the union of its
 * ranges).  The W units in group-major order are cut into num_splits
 * contiguous pieces, piece c = units [floor(c*W/num_splits),
 * floor((c+1)*W/num_splits)); schedule [num_splits + 1][2] int32 receives
 * (g, t) of the first unit of each piece and (ceil(Sq/4), 0) for the end (or
 * for a piece that starts at W).  Requires 1 <= num_splits <= 65536 and
 * Sq <= 32768.
 */
int64_t mqa_logits_metadata_size(int32_t num_splits);  /* int32 count */
mqa_status mqa_logits_metadata(const int32_t* k_start, const int32_t* k_end,
                               int32_t sq, int32_t skv, int32_t num_splits,
                               int32_t* schedule, hipStream_t stream);

/*
 * Row offsets of the compressed layout ("Compressed Logits" in the DeepGEMM
 * MQA-logits article: only [seq_k_start, seq_k_end) of each row is stored).
 * Writes the exclusive prefix sum of the clamped row lengths e_i - s_i:
 * row_offsets [Sq + 1] int64, row_offsets[0] = 0, row_offsets[Sq] = total.
 */
mqa_status mqa_logits_compressed_offsets(const int32_t* k_start, const int32_t* k_end,
                                         int32_t sq, int32_t skv,
                                         int64_t* row_offsets, hipStream_t stream);

/*
 * Compressed logits: entry (i, j), s_i <= j < e_i, is written to
 * logits_packed[row_offsets[i] + (j - s_i)]; nothing else is written.
 * logits_packed holds row_offsets[Sq] elements of logits_type (aligned to
 * the element size).  Other arguments as mqa_logits.
 */
mqa_status mqa_logits_compressed(mqa_dtype dt,
                                 const void* q, const uint8_t* q_sf,
                                 const void* kv, const uint8_t* kv_sf,
                                 const float* kv_scale, const void* weights,
                                 const int32_t* k_start, const int32_t* k_end,
                                 const int64_t* row_offsets, void* logits_packed,
                                 int32_t sq, int32_t skv, int32_t h, int32_t d,
                                 mqa_float weights_type, mqa_float logits_type,
                                 const int32_t* schedule, int32_t num_splits,
                                 mqa_precision precision, hipStream_t stream);

/*
 * Top-k over logits rows: the sparse-attention indices that consume the
 * logits ("FlashMLA" page, flash_mla_with_kvcache parameters: `indices` of
 * shape (batch_size, seq_len_q, topk), invalid entries -1; get_mla_metadata's
 * `topk` sparsity parameter).
 *   logits   [Sq, logits_stride] of logits_type (the output of mqa_logits or,
 *            with rows b*next_n + t, of paged_mqa_logits)
 *   k_start, k_end [Sq] int32, both or neither: row i's range is
 *            [clamp(k_start, 0, Skv), clamp(k_end, start, Skv)); without them
 *            every row is [0, Skv)
 *   indices  [Sq, indices_stride] int32, indices_stride >= topk
 * Row i's candidates are the columns of its range whose logit is not -inf.
 * indices[i, :] receives the columns of its topk largest candidates in
 * ascending column order, then -1 up to topk when the row has fewer.  Order:
 * larger values first, -0 below +0 (IEEE 754 total order of the bit
 * patterns), equal values by smaller column, so the selected set is unique.
 * Requires topk >= 1.
 */
mqa_status mqa_logits_topk(const void* logits, mqa_float logits_type, int64_t logits_stride,
                           const int32_t* k_start, const int32_t* k_end,
                           int32_t sq, int32_t skv, int32_t topk,
                           int32_t* indices, int64_t indices_stride, hipStream_t stream);

/*
 * Paged schedule ("Implementing Paged MQA Logits Computation for Decoding" in
 * the DeepGEMM MQA-logits article: a metadata call made once per decoding
 * step from context_lens, block_kv and the SM count; "[PR #314] fix: SM90
 * paged MQA logits IMA on next_n=4", a97b74d Root cause / Fix: one entry per
 * worker plus one, decoded as (query index, KV block index)).
 *
 * Work units: sequence b owns n_b = ceil(min(ctx_b, max_context_len) /
 * block_size) units (b, 0) .. (b, n_b - 1), one KV block for all next_n query
 * rows of b.  The W units in sequence-major order are cut into num_splits
 * contiguous pieces; piece c = units [floor(c*W/num_splits),
 * floor((c+1)*W/num_splits)).  schedule [num_splits + 1][2] int32 receives
 * (b, blk) of the first unit of each piece, and (batch, 0) for the end (or for
 * a piece that starts at W).  The same num_splits must be passed to
 * paged_mqa_logits.  Requires 1 <= batch <= 8192, 1 <= next_n <= 16,
 * block_size in {16, 32, 64}, 1 <= num_splits <= 65536.
 */
int64_t paged_mqa_logits_metadata_size(int32_t num_splits);  /* int32 count */
mqa_status paged_mqa_logits_metadata(const int32_t* context_lens, int32_t batch,
                                     int32_t next_n, int32_t block_size,
                                     int32_t max_context_len, int32_t num_splits,
                                     int32_t* schedule, hipStream_t stream);

/*
 * Paged decode logits (the paged path of the DeepGEMM MQA-logits article;
 * next_n query tokens per sequence as in PR #314, 12cb7c0).
 *   q        [batch*next_n, H, D] (fp4: D/2 bytes); row r = b*next_n + t
 *   q_sf     [batch*next_n, H, D/32] or NULL
 *   kv_pool  [num_blocks, block_size, D] (fp4: D/2 bytes)
 *   kv_sf_pool [num_blocks, block_size, D/32] or NULL
 *   kv_scale_pool [num_blocks, block_size] fp32 (FP8 only, else NULL)
 *   weights  [batch*next_n, H] of weights_type
 *   context_lens [batch] int32: tokens of sequence b including its next_n new
 *            ones; logical token j of b is slot j % block_size of physical
 *            block block_table[b * block_table_stride + j / block_size]
 *            (row b is read up to entry ceil(min(ctx_b, max_context_len) /
 *            block_size); ids are clamped to [0, num_blocks); the Python
 *            binding requires rows of ceil(max_context_len / block_size))
 *   schedule from paged_mqa_logits_metadata with the same arguments
 *   logits   [batch*next_n, logits_stride] of logits_type, logits_stride >=
 *            max_context_len (even for bf16; the pointer 4-byte aligned).
 *            Row b*next_n + t covers keys
 *            [0, clamp(ctx_b - next_n + t + 1, 0, min(ctx_b, max_context_len)));
 *            with clean_logits the rest of [0, max_context_len) is -inf.
 *   precision: mqa_precision above (the paged kernel evaluates ReLU per head
 *            in both modes).
 */
mqa_status paged_mqa_logits(mqa_dtype dt,
                            const void* q, const uint8_t* q_sf,
                            const void* kv_pool, const uint8_t* kv_sf_pool,
                            const float* kv_scale_pool, const void* weights,
                            const int32_t* context_lens,
                            const int32_t* block_table, int64_t block_table_stride,
                            const int32_t* schedule,
                            void* logits, int64_t logits_stride,
                            int32_t batch, int32_t next_n, int32_t h, int32_t d,
                            int32_t block_size, int32_t num_blocks,
                            int32_t max_context_len, int32_t num_splits,
                            int32_t clean_logits, mqa_float weights_type,
                            mqa_float logits_type, mqa_precision precision,
                            hipStream_t stream);

/* Compute units of a device (the get_num_sms analogue of the DeepGEMM
 * article's paged example); negative on error. */
int32_t mqa_num_cus(int32_t device);

/* A good num_splits for paged_mqa_logits on a device: 4 workers per compute
 * unit, all resident at once (a worker is one wave, or two waves that split
 * 64 heads, whose registers allow two workers per SIMD); negative on error. */
int32_t paged_mqa_logits_default_splits(int32_t device);

/* Thread-local description of the last non-OK status ("" if none). */
const char* mqa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MQA_LOGITS_H */
