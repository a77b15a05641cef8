/*
 * kvrec.h - C ABI of the MI355X (gfx950) paged KV-record codec.
 *
 * Two operations on a paged uint8 KV cache holding one 512-dim MLA latent
 * per token:
 *
 *   kvrec_insert  fused fp32 RoPE on the 64 tail dims + MXFP8 (or legacy)
 *                 quantisation + paged store of the token's record
 *                 (kvrec_insert_ex adds the compressed-KV options;
 *                 kvrec_insert_full writes the non-packed bf16 / fp8 caches);
 *   kvrec_gather  the inverse: paged read + dequantisation to bf16 rows;
 *   kvrec_qnorm_rope_insert  the attention write: q RMSNorm + RoPE for every
 *                 head, fused with kvrec_insert in one launch;
 *   kvrec_expand_candidates  the sparse indexer's candidate-block expansion
 *                 into the sorted sparse block indices that select what the
 *                 attention reads.
 *
 * Sources (page titles; sections named as on the pages):
 *   [MXFP8 record] vLLM PR #56893 report, "[Model][DSv4.1] Store the whole KV
 *                  in MXFP8 (FlashMLA V4.1 record)"
 *   [KV-only op]   vLLM PR #56441 report, "[Perf][DSpark] Add KV-only context
 *                  insertion across V4.1 cache formats"
 *   [FlashMLA]     article page "deepseek-ai/FlashMLA" (ssnai.com)
 *   [Sparse indexer] vLLM PR #56254 report, "[DSA] Wire DeepGEMM sparse MQA
 *                  logits into the DeepSeek V4.1 indexer"
 *
 * Conventions for every call:
 *   - Pointers marked (device) are HIP device memory of the current device;
 *     kvrec_cache is a host struct describing device memory.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL is the legacy
 *     default stream). The library allocates nothing, keeps no state and
 *     never synchronises. The caller owns every buffer.
 *   - Every argument check runs on the host before any launch; on error the
 *     call returns a negative kvrec_status and nothing is launched or
 *     written. The library never throws or aborts across this ABI.
 *   - A call over more than 2^21 waves of work (2^22 tokens of an insert,
 *     2^22 gather rows, 2^21 expansion rows, fewer attention-write tokens)
 *     runs as several kernel launches on `stream`, one per consecutive slice
 *     of the rows, in order. If a later launch fails (KVREC_ERR_HIP), the
 *     slices before it have been enqueued.
 *   - Device-resident values are not inspected on the host. Preconditions
 *     the caller keeps: non-negative slots distinct within one insert; kv
 *     finite with |x| < 2^127 (so the rotation cannot overflow), except
 *     that NaN (never an infinity) is allowed in kvrec_insert_ex with
 *     sanitize_nans = 1; kv, out and token_indices do not overlap the cache. As a memory-safety guard the
 *     kernels skip a token whose slot is >= num_blocks * block_size or whose
 *     position is outside [0, max_pos), and gather a zero row for an index
 *     >= num_blocks * block_size.
 */
#ifndef KVREC_H
#define KVREC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Latent width and rotated tail ([MXFP8 record] 功能与动机; [KV-only op]
 * 实现拆解 1: kv is bf16 [tokens, 512], cos_sin_cache fp32 [max_pos, 64]). */
#define KVREC_HEAD_DIM 512
#define KVREC_ROPE_DIM 64

/* Record widths in bytes per token, which also select the format
 * ([MXFP8 record] 功能与动机 and 实现拆解 4; [KV-only op] 实现拆解 1: the
 * packed cache's last dimension must be 528 or 584):
 *   528  MXFP8 record: 512 e4m3fn codes (RoPE dims rotated, then quantised)
 *        + 16 UE8M0 scales, one per 32 dims; page alignment 512 B.
 *   584  legacy record: 448 e4m3fn codes of the NoPE dims + 64 rotated RoPE
 *        dims as bf16 (576 B data row) + 7 UE8M0 scales over 64-dim groups
 *        + 1 pad byte (8 B scale row); page alignment 576 B. */
#define KVREC_RECORD_MXFP8 528
#define KVREC_RECORD_LEGACY 584

/* Non-packed caches of the KV-only op ([KV-only op] 实现拆解 1: a bf16 cache,
 * or an fp8 e4m3fn cache with one float32 per-tensor scale; 512 elements per
 * token), written by kvrec_insert_full only. Widths in bytes per token:
 *   1024  bf16 row: the 512 dims as bf16 (rotated tail rounded to nearest
 *         even; dims 0..447 are the input bits).
 *   512   fp8 row: the 512 dims as e4m3fn codes of the fp32 quotient
 *         r / scale, nearest even, saturated to +-448.
 * A slot's row sits at page + (slot % block_size) * width; there is no scale
 * region. Page alignment 16 B. */
#define KVREC_RECORD_BF16 1024
#define KVREC_RECORD_FP8 512

typedef enum kvrec_status {
  KVREC_OK = 0,
  KVREC_ERR_NULL = -1,        /* a required pointer is NULL               */
  KVREC_ERR_RECORD = -2,      /* record not one the call takes, or !=
                                 the cache's record                       */
  KVREC_ERR_BLOCK_SIZE = -3,  /* block_size < 1, != cache's block_size, or
                                 block_size * record > 2^31               */
  KVREC_ERR_PAGE_STRIDE = -4, /* page stride not a multiple of the record's
                                 alignment, or < block_size * record      */
  KVREC_ERR_ALIGNMENT = -5,   /* a pointer is not aligned as stated below */
  KVREC_ERR_SIZE = -6,        /* negative count, max_pos < 1, or a size
                                 beyond what the kernels index            */
  KVREC_ERR_HIP = -7,         /* the HIP launch reported an error         */
  KVREC_ERR_OPTION = -8,      /* an insert option is out of range         */
  KVREC_ERR_OVERLAP = -9      /* an output partly overlaps an input       */
} kvrec_status;

/* A paged cache: num_blocks pages, page_stride bytes apart, each holding
 * block_size records laid out as a data region (block_size rows of 512 B, or
 * 576 B for the legacy record) followed by a scale region (block_size rows of
 * 16 B, or 8 B) and then padding up to page_stride ([MXFP8 record] 实现拆解 4
 * and 关键源码片段: data at page + off*512, scales at page + block*512 +
 * off*16). The non-packed caches have the data region only. A token in slot
 * s lives in page s / block_size at offset s % block_size. */
typedef struct kvrec_cache {
  void *base;          /* (device) byte 0 of page 0; 16-B aligned          */
  int64_t num_blocks;  /* pages, >= 0; num_blocks * block_size <= 2^30   */
  int64_t page_stride; /* bytes between pages; a multiple of 512 (528),
                          576 (584) or 16 (1024, 512), and >= block_size *
                          record                                           */
  int32_t block_size;  /* tokens per page, >= 1; block_size * record
                          <= 2^31                                          */
  int32_t record;      /* 528, 584, 1024 or 512                            */
} kvrec_cache;

/* hipStream_t, passed opaquely so this header needs no HIP headers. */
typedef void *kvrec_stream;

/* Page stride for a record and block size: block_size * record rounded up
 * to the record's alignment (512, 576 or 16). Host-only, pure.
 * Returns KVREC_OK and writes *page_stride_out, or KVREC_ERR_NULL,
 * KVREC_ERR_RECORD, KVREC_ERR_BLOCK_SIZE. */
int kvrec_page_stride(int32_t record, int32_t block_size, int64_t *page_stride_out);

/* Insert num_tokens tokens ([KV-only op] 实现拆解 1 and 2: kv, k_cache,
 * slot_mapping, positions, cos_sin_cache, cache block size; the record is
 * read from the cache's last dimension).
 *
 *   kv            (device) bf16 [num_tokens, 512], rows contiguous; 16-B
 *                 aligned; read only.
 *   num_tokens    0 .. 2^30; 0 returns KVREC_OK without a launch.
 *   k_cache       host descriptor of the cache written in place.
 *   slot_mapping  (device) int64 [num_tokens]; 8-B aligned. A negative slot
 *                 skips its token: nothing is written for it.
 *   positions     (device) int64 [num_tokens]; 8-B aligned; the row of
 *                 cos_sin_cache for each token.
 *   cos_sin_cache (device) fp32 [max_pos, 64]: 32 cos values then 32 sin
 *                 values per row; 16-B aligned.
 *   max_pos       rows of cos_sin_cache, 1 .. 2^30.
 *   block_size    must equal k_cache->block_size (cross-check, as the page's
 *                 op keeps k_cache.size(1) == cache_block_size).
 *   record        must equal k_cache->record.
 *
 * Per token, in order: RoPE on dims 448..511 in fp32 with pairs
 * (448+i, 480+i), r1 = x1*c - x2*s and r2 = x2*c + x1*s, each product and
 * the add rounded separately (no fused multiply-add); dims 0..447 unchanged.
 * MXFP8: for each 32-dim group, amax = max |r|, e = the smallest integer with
 * amax <= 448 * 2^e clamped to [-127, 127] (e = 0 when amax == 0), scale
 * byte e + 127, codes = e4m3fn(r * 2^-e) rounded to nearest even. Legacy: the
 * same over seven 64-dim NoPE groups, and the rotated tail as bf16 (nearest
 * even). Only the token's record bytes are written: page padding, other
 * slots and skipped tokens keep their bytes.
 * ([MXFP8 record] 功能与动机, 实现拆解 3 and 关键源码片段.) */
int kvrec_insert(const void *kv, int64_t num_tokens, const kvrec_cache *k_cache,
                 const int64_t *slot_mapping, const int64_t *positions,
                 const float *cos_sin_cache, int64_t max_pos, int32_t block_size,
                 int32_t record, kvrec_stream stream);

/* Options of kvrec_insert_ex. kvrec_insert is kvrec_insert_ex with
 * {KVREC_ROPE_NEOX, 1, 0.0f, 0}. The other settings follow the compressed-KV
 * insert printed in [MXFP8 record] 关键源码片段 (its
 * "_rope_quant_insert_mxfp8_kernel") and the K insert without RoPE of
 * [MXFP8 record] 实现拆解 4.
 *   rope            KVREC_ROPE_NEOX: pairs (448+i, 480+i), dims 0..447 untouched.
 *                   KVREC_ROPE_INTERLEAVED: neighbour pairs (2p, 2p+1); pairs
 *                   224..255 rotate with cos row[p-224], sin row[32+p-224];
 *                   the NoPE pairs go through the same products with
 *                   (cos, sin) = (1, 0) (a -0 whose partner is negative turns
 *                   +0; a NaN spreads to its partner).
 *                   KVREC_ROPE_NONE: no rotation; the table is not read.
 *   compress_ratio  R in [1, 2^30]: only tokens with (position + 1) % R == 0
 *                   are written, rotated with table row position / R * R.
 *   amax_floor      finite, >= 0: each group's amax is raised to it before
 *                   the exponent is chosen (the excerpt uses 1e-4; 0 = none).
 *   sanitize_nans   0 or 1: rotated NaNs become +0 before quantisation;
 *                   with 1, kv may hold NaNs (never infinities). */
typedef enum kvrec_rope {
  KVREC_ROPE_NEOX = 0,
  KVREC_ROPE_INTERLEAVED = 1,
  KVREC_ROPE_NONE = 2
} kvrec_rope;

typedef struct kvrec_insert_options {
  int32_t rope;
  int32_t compress_ratio;
  float amax_floor;
  int32_t sanitize_nans;
} kvrec_insert_options;

/* kvrec_insert with options (NULL = the defaults). Same arguments, layout
 * and errors as kvrec_insert, plus KVREC_ERR_OPTION for an option out of
 * range. With rope == KVREC_ROPE_NONE the table is not read and
 * cos_sin_cache may be NULL (nor is it checked); with compress_ratio == 1 as
 * well, positions are not read either, may be NULL, and skip no token even
 * when given and out of range (positions and max_pos are then ignored). */
int kvrec_insert_ex(const void *kv, int64_t num_tokens, const kvrec_cache *k_cache,
                    const int64_t *slot_mapping, const int64_t *positions,
                    const float *cos_sin_cache, int64_t max_pos, int32_t block_size,
                    int32_t record, const kvrec_insert_options *options,
                    kvrec_stream stream);

/* Insert into a non-packed cache (record KVREC_RECORD_BF16 or
 * KVREC_RECORD_FP8): the KV-only op's bf16 and fp8 branches ([KV-only op]
 * 实现拆解 1, which requires a float32 scalar scale for the fp8 cache).
 * Arguments, skip rules and errors as kvrec_insert, with the NeoX rotation
 * and no options, plus:
 *   fp8_scale  (device) one fp32, 4-B aligned, read on the device: the
 *              per-tensor scale of the fp8 cache (stored code * scale
 *              approximates the value). Required (KVREC_ERR_NULL) for
 *              record 512; must be NULL (KVREC_ERR_OPTION) for record 1024.
 *              The caller keeps it positive and finite.
 * The packed calls (kvrec_insert, kvrec_insert_ex, kvrec_gather) refuse
 * these records with KVREC_ERR_RECORD, and this call refuses 528 / 584. */
int kvrec_insert_full(const void *kv, int64_t num_tokens, const kvrec_cache *k_cache,
                      const int64_t *slot_mapping, const int64_t *positions,
                      const float *cos_sin_cache, int64_t max_pos, int32_t block_size,
                      int32_t record, const float *fp8_scale, kvrec_stream stream);

/* The attention write: the q side of the QNorm op ([KV-only op] 实现拆解 1
 * lists its q_in, q_head_padded, eps and apply_q_norm arguments; [MXFP8
 * record] 关键源码片段 calls it with padded_heads and eps) fused with
 * kvrec_insert, in one launch. The pages name these arguments only; the
 * readings: every head of every token is processed (the slot only decides
 * the cache write), the norm is an RMSNorm over the head's 512 dims with no
 * weight, and q is rotated like the KV latent (NeoX pairs of dims 448..511,
 * the token's table row).
 *
 *   q_in          (device) bf16 [num_tokens, num_heads, 512], contiguous,
 *                 16-B aligned.
 *   q_out         (device) same shape; q_in itself (in place) or a buffer
 *                 that does not overlap it (KVREC_ERR_OVERLAP otherwise).
 *   num_heads     1 .. 1024 (the padded head count); num_tokens * num_heads
 *                 <= 2^30.
 *   eps           with apply_q_norm: finite and > 0 (KVREC_ERR_OPTION).
 *   apply_q_norm  0: rotation only; 1: y = x / sqrt(mean(x^2) + eps) first.
 *   the rest      as kvrec_insert (packed records 528 / 584 only).
 *
 * Per head, in fp32: the sum of squares (products and sums rounded one by
 * one, in a fixed order), inv = an approximation of 1 / sqrt(sum / 512 +
 * eps) within 1 ulp, y = x * inv, the rotation as in kvrec_insert, and bf16
 * nearest even. The sum order is not the oracle's, so q_out agrees with the
 * exact result to within the error bound of this arithmetic, not bit for
 * bit; the cache bytes are exactly those of kvrec_insert. A token whose
 * position is outside [0, max_pos) leaves its q_out rows unwritten. */
int kvrec_qnorm_rope_insert(const void *q_in, void *q_out, int32_t num_heads, float eps,
                            int32_t apply_q_norm, const void *kv, int64_t num_tokens,
                            const kvrec_cache *k_cache, const int64_t *slot_mapping,
                            const int64_t *positions, const float *cos_sin_cache,
                            int64_t max_pos, int32_t block_size, int32_t record,
                            kvrec_stream stream);

/* Candidate-block expansion ([Sparse indexer] 关键源码片段: the per-row
 * program _expand_candidates_kernel and candidate_blocks_to_sparse_indices).
 * For each of `rows` rows, in the page's order:
 *   - take the row's K candidate block ids; with ratio 2 each candidate c
 *     becomes the two sparse blocks 2c and 2c + 1 (a candidate block of
 *     2 * SBK tokens split in two);
 *   - keep the blocks b with 0 <= b < ceil(max(ke - ks, 0) / SBK);
 *   - sort them ascending (duplicates kept) and add base = ks / SBK;
 *   - write them to the row's K * ratio outputs, padding after the n_valid
 *     kept ones with the last kept block + base (base when none is kept);
 *   - end = (n_valid - 1) * SBK + min(max(ke - (last * SBK + ks), 1), SBK),
 *     or 0 when nothing is kept (only the last block can be partial).
 * Integer arithmetic is exact (no int32 wrap of intermediate values). For
 * rows with ke - ks > 2^31 - SBK this differs from the page's int32 program,
 * whose ke - ks + SBK - 1 wraps negative there so that it keeps no block:
 * here such a row keeps the blocks that cover [ks, ke), as any shorter row.
 *
 *   candidate_blocks (device) int32, row r at r * cand_stride (elements),
 *                    K entries; cand_stride >= K.
 *   row_ks, row_ke   (device) int32, row r at r * ks_stride / r * ke_stride
 *                    (>= 1): the row's KV range [ks, ke). The caller keeps
 *                    ks >= 0 and ke >= 0.
 *   rows             0 .. 2^30; 0 returns KVREC_OK without a launch.
 *   num_candidates   K, a power of two, K * ratio <= 1024 (KVREC_ERR_SIZE).
 *   ratio            1 or 2; sparse_block (SBK) 8 or 16 (KVREC_ERR_OPTION).
 *   sparse_indices   (device) int32 out, row r at r * sparse_stride, K * ratio
 *                    entries; sparse_stride >= K * ratio.
 *   end              (device) int32 out, row r at r * end_stride (>= 1).
 * All pointers 4-B aligned; outputs must not overlap the inputs. */
int kvrec_expand_candidates(const int32_t *candidate_blocks, int64_t cand_stride,
                            const int32_t *row_ks, int64_t ks_stride, const int32_t *row_ke,
                            int64_t ke_stride, int64_t rows, int32_t num_candidates,
                            int32_t ratio, int32_t sparse_block, int32_t *sparse_indices,
                            int64_t sparse_stride, int32_t *end, int64_t end_stride,
                            kvrec_stream stream);

/* Gather num_indices records back to bf16 rows ([MXFP8 record] 实现拆解 4:
 * one gather parameterised by the record; [FlashMLA]: index =
 * page * block_size + offset, -1 marks an invalid entry).
 *
 *   k_cache        host descriptor of the cache; read only.
 *   token_indices  (device) int32 [num_indices]; 4-B aligned. A negative
 *                  index gives a row of +0.
 *   num_indices    0 .. 2^30; 0 returns KVREC_OK without a launch.
 *   out            (device) bf16 [num_indices, 512]; 16-B aligned; written.
 *
 * Element d of a valid row is the bf16 nearest to e4m3fn(code_d) *
 * 2^(scale - 127) (exact whenever the scale byte is >= 3); the RoPE dims
 * come back rotated. Legacy record: dims 448..511 are the stored bf16. */
int kvrec_gather(const kvrec_cache *k_cache, const int32_t *token_indices,
                 int64_t num_indices, void *out, kvrec_stream stream);

/* Static string naming a kvrec_status (never NULL). */
const char *kvrec_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* KVREC_H */
