/*
 * kvrec_oracle.h - plain CPU reference of the paged KV-record codec.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. The product path (libkvrec.so)
 * never links, loads or calls it, and shares no code, header, table or
 * helper with it.
 *
 * Every function is a direct, slow statement of what the pages define:
 *   [MXFP8 record]  vLLM PR #56893 report, "[Model][DSv4.1] Store the whole KV
 *                   in MXFP8 (FlashMLA V4.1 record)"
 *   [KV-only op]    vLLM PR #56441 report, "[Perf][DSpark] Add KV-only context
 *                   insertion across V4.1 cache formats"
 *   [FlashMLA]      article page "deepseek-ai/FlashMLA" (ssnai.com)
 *   [Sparse indexer] vLLM PR #56254 report, "[DSA] Wire DeepGEMM sparse MQA
 *                   logits into the DeepSeek V4.1 indexer"
 * Where the pages leave a step open, the reading taken is stated at the
 * function. All integers are host-endian (little-endian x86-64).
 */
#ifndef KVREC_ORACLE_H
#define KVREC_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- element codecs ---------------------------------------------------- */

/* Exact real value of an OCP e4m3fn code (NaN for 0x7F / 0xFF). */
double orc_e4m3_value(uint8_t code);

/* e4m3fn code nearest to y, ties to the even code, |y| >= 448 -> +-448. */
uint8_t orc_e4m3_encode(double y);

/* bfloat16 bits nearest to x, ties to even, beyond the largest finite
 * rounding threshold -> +-inf. */
uint16_t orc_bf16_round(double x);

/* Smallest integer e with amax <= 448 * 2^e, clamped to [-127, 127];
 * amax == 0 gives 0. */
int orc_scale_exponent(float amax);

/* ---- the operations ---------------------------------------------------- */

/* Insert n tokens into a host copy of the paged cache.
 *   kv            bf16 bits [n, 512], row-major
 *   cache         byte 0 of page 0; num_blocks pages page_stride bytes apart
 *   block_size    tokens per page
 *   record        528 (MXFP8 record) or 584 (legacy record)
 *   slot_mapping  [n] int64; negative -> token skipped
 *   positions     [n] int64; row of cos_sin_cache to use
 *   cos_sin_cache fp32 [max_pos, 64]: 32 cos values then 32 sin values
 * Returns 0, or -1 if record is not 528/584. */
int orc_insert(const uint16_t *kv, int64_t n, uint8_t *cache,
               int64_t num_blocks, int64_t page_stride, int32_t block_size,
               int32_t record, const int64_t *slot_mapping,
               const int64_t *positions, const float *cos_sin_cache,
               int64_t max_pos);

/* Options of the insert. The defaults (NEOX, 1, 0.0f, 0) are orc_insert.
 * The other settings follow the compressed-KV insert printed in
 * [MXFP8 record] 关键源码片段 (its "_rope_quant_insert_mxfp8_kernel"). */
enum { ORC_ROPE_NEOX = 0, ORC_ROPE_INTERLEAVED = 1, ORC_ROPE_NONE = 2 };
typedef struct orc_insert_options {
  int32_t rope;           /* pairing of the 64 rotated dims, or no rotation  */
  int32_t compress_ratio; /* >= 1: write only tokens with (pos+1) % R == 0,
                             rotating with cos/sin row pos / R * R         */
  float amax_floor;       /* group amax = max(amax, floor); 0 = no floor     */
  int32_t sanitize_nans;  /* 1: rotated NaN -> +0, scale byte capped at 254 */
} orc_insert_options;

int orc_insert_ex(const uint16_t *kv, int64_t n, uint8_t *cache, int64_t num_blocks,
                  int64_t page_stride, int32_t block_size, int32_t record,
                  const int64_t *slot_mapping, const int64_t *positions,
                  const float *cos_sin_cache, int64_t max_pos,
                  const orc_insert_options *opts);

/* Non-packed caches [KV-only op, 实现拆解 1]: record = bytes per slot.
 *   ORC_RECORD_BF16  512 bf16 elements, little-endian
 *   ORC_RECORD_FP8   512 e4m3fn codes of fl(r / fp8_scale), saturated
 * Rows sit at page * page_stride + (slot % block_size) * record; there is no
 * scale region. The rotation is the NeoX one of orc_insert; fp8_scale is
 * read only for ORC_RECORD_FP8. Returns 0, or -1 for another record. */
enum { ORC_RECORD_BF16 = 1024, ORC_RECORD_FP8 = 512 };
int orc_insert_full(const uint16_t *kv, int64_t n, uint8_t *cache, int64_t num_blocks,
                    int64_t page_stride, int32_t block_size, int32_t record,
                    const int64_t *slot_mapping, const int64_t *positions,
                    const float *cos_sin_cache, int64_t max_pos, float fp8_scale);

/* q side of the attention write: per token and head (q bf16 [n, heads, 512]),
 * y = x / sqrt(mean(x^2) + eps) if apply_norm (else y = x), the NeoX
 * rotation of dims 448..511 with the token's table row, and the bf16 nearest
 * to each exact result (binary64 arithmetic, one rounding). Tokens with a
 * position outside [0, max_pos) leave q_out unwritten. q_out may be q_in. */
void orc_qnorm_rope(const uint16_t *q_in, int64_t n, int32_t heads, const int64_t *positions,
                    const float *cos_sin_cache, int64_t max_pos, double eps, int32_t apply_norm,
                    uint16_t *q_out);

/* Gather n records back to bf16 rows.
 *   token_indices [n] int32, page * block_size + offset; negative -> zeros
 *   out           bf16 bits [n, 512]
 * Returns 0, or -1 if record is not 528/584. */
int orc_gather(const uint8_t *cache, int64_t num_blocks, int64_t page_stride,
               int32_t block_size, int32_t record,
               const int32_t *token_indices, int64_t n, uint16_t *out);

/* Candidate-block expansion of the sparse indexer ([Sparse indexer]
 * 关键源码片段, _expand_candidates_kernel), for `rows` rows:
 *   cand        int32 [rows, K] (row stride cand_stride elements)
 *   row_ks/ke   int32 per row (strides ks_stride / ke_stride): the row's KV
 *               range [ks, ke)
 *   ratio       1 or 2 (2 splits a candidate c into sparse blocks 2c, 2c+1)
 *   sparse_block SBK, tokens per sparse block
 *   sparse      int32 [rows, K * ratio] out: the sorted kept blocks + ks/SBK,
 *               padded with the last one
 *   end         int32 per row out: valid sparse token columns
 * Returns 0, or -1 for a bad K / ratio / SBK (or no memory). */
int orc_expand_candidates(const int32_t *cand, int64_t cand_stride, const int32_t *row_ks,
                          int64_t ks_stride, const int32_t *row_ke, int64_t ke_stride,
                          int64_t rows, int32_t num_candidates, int32_t ratio,
                          int32_t sparse_block, int32_t *sparse, int64_t sparse_stride,
                          int32_t *end, int64_t end_stride);

/* ---- batch forms of the element codecs, for the pin tests -------------- */

void orc_e4m3_encode_f32(const float *y, int64_t n, uint8_t *out);
void orc_e4m3_encode_bits(uint32_t first_bits, int64_t n, uint8_t *out);
void orc_e4m3_value_all(double *out256);
void orc_bf16_round_f32(const float *x, int64_t n, uint16_t *out);
void orc_scale_exponent_f32(const float *amax, int64_t n, int32_t *out);
void orc_rope_rows(const uint16_t *kv, int64_t n, const int64_t *positions,
                   const float *cos_sin_cache, float *out);
void orc_rope_rows_ex(const uint16_t *kv, int64_t n, const int64_t *positions,
                      const float *cos_sin_cache, const orc_insert_options *opts, float *out);

#ifdef __cplusplus
}
#endif

#endif /* KVREC_ORACLE_H */
