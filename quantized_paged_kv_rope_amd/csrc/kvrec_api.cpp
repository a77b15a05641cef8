// kvrec_api.cpp - the C ABI declared in include/kvrec.h: argument checks on
// the host, then the kernel launch (one per slice of at most 2^21 waves) on
// the caller's stream.
//
// Checks follow the validation list of the page's KV-only op ([KV-only op]
// 实现拆解 1: dtype/shape/stride/record-width checks at the op's entry, and
// nothing runs on failure), restated for plain pointers: the record width
// selects the kernel, the block size is cross-checked against the cache, the
// page stride must be a multiple of the record's page alignment (512 B for
// the 528 B record, 576 B for the 584 B record: [MXFP8 record] 功能与动机;
// 16 B, the width of one vector store, for the non-packed rows), and the fp8
// cache needs its scale.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <hip/hip_runtime.h>

#include "kvrec.h"
#include "kvrec_launch.h"

namespace {

// Rows and slots per call: indices stay 32-bit on the device. Calls of more
// rows than one launch takes run as several launches (kvrec::kMaxLaunchWaves).
constexpr int64_t kMaxCount = int64_t{1} << 30;
constexpr int64_t kMaxPos = int64_t{1} << 30;    // cos/sin rows (a 256 GB table); pos + 1 < 2^31
constexpr int32_t kMaxHeads = 1024;              // q heads of the attention write
constexpr int32_t kMaxExpanded = 1024;           // K * RATIO of the candidate expansion

bool misaligned(const void *p, uintptr_t align) {
  return (reinterpret_cast<uintptr_t>(p) & (align - 1)) != 0;
}

int64_t record_alignment(int32_t record) {
  return record == KVREC_RECORD_MXFP8 ? 512 : record == KVREC_RECORD_LEGACY ? 576 : 16;
}

bool packed_record(int32_t record) {
  return record == KVREC_RECORD_MXFP8 || record == KVREC_RECORD_LEGACY;
}

bool full_record(int32_t record) {
  return record == KVREC_RECORD_BF16 || record == KVREC_RECORD_FP8;
}

bool known_record(int32_t record) { return packed_record(record) || full_record(record); }

// In-page byte offsets are computed in 32 bits on the device; a page of
// block_size records must stay below 2^31 bytes.
constexpr int64_t kMaxPageBytes = int64_t{1} << 31;

// Division by an invariant block size with a multiply-high (Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994):
// with l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1, the quotient of
// n by d is (umulhi(n, m) + n) >> l for every n < 2^31 (the sum cannot
// overflow 32 bits there).
void division_magic(uint32_t d, uint32_t *magic, uint32_t *shift) {
  uint32_t l = 0;
  while ((uint64_t{1} << l) < d) ++l;
  *magic = static_cast<uint32_t>(((uint64_t{1} << 32) * ((uint64_t{1} << l) - d)) / d + 1);
  *shift = l;
}

// Checks a cache descriptor; on success fills the kernels' geometry.
int check_cache(const kvrec_cache *c, kvrec::CacheGeom *g) {
  if (c == nullptr || c->base == nullptr) return KVREC_ERR_NULL;
  if (!known_record(c->record)) return KVREC_ERR_RECORD;
  if (c->block_size < 1) return KVREC_ERR_BLOCK_SIZE;
  if (c->num_blocks < 0) return KVREC_ERR_SIZE;
  const int64_t page_bytes = static_cast<int64_t>(c->block_size) * c->record;
  if (page_bytes > kMaxPageBytes) return KVREC_ERR_BLOCK_SIZE;
  if (c->page_stride < page_bytes || c->page_stride % record_alignment(c->record) != 0)
    return KVREC_ERR_PAGE_STRIDE;
  if (c->num_blocks > kMaxCount / c->block_size) return KVREC_ERR_SIZE;
  if (c->num_blocks > INT64_MAX / c->page_stride) return KVREC_ERR_SIZE;
  if (misaligned(c->base, 16)) return KVREC_ERR_ALIGNMENT;
  g->base = static_cast<uint8_t *>(c->base);
  g->page_stride = c->page_stride;
  g->block_size = static_cast<uint32_t>(c->block_size);
  g->total_slots = static_cast<uint32_t>(c->num_blocks * c->block_size);
  division_magic(g->block_size, &g->div_magic, &g->div_shift);
  return KVREC_OK;
}

}  // namespace

extern "C" {

int kvrec_page_stride(int32_t record, int32_t block_size, int64_t *page_stride_out) {
  if (page_stride_out == nullptr) return KVREC_ERR_NULL;
  if (!known_record(record)) return KVREC_ERR_RECORD;
  if (block_size < 1 || static_cast<int64_t>(block_size) * record > kMaxPageBytes)
    return KVREC_ERR_BLOCK_SIZE;
  const int64_t align = record_alignment(record);
  const int64_t raw = static_cast<int64_t>(block_size) * record;
  *page_stride_out = (raw + align - 1) / align * align;
  return KVREC_OK;
}

int kvrec_insert(const void *kv, int64_t num_tokens, const kvrec_cache *k_cache,
                 const int64_t *slot_mapping, const int64_t *positions,
                 const float *cos_sin_cache, int64_t max_pos, int32_t block_size,
                 int32_t record, kvrec_stream stream) {
  return kvrec_insert_ex(kv, num_tokens, k_cache, slot_mapping, positions, cos_sin_cache, max_pos,
                         block_size, record, nullptr, stream);
}

int kvrec_insert_ex(const void *kv, int64_t num_tokens, const kvrec_cache *k_cache,
                    const int64_t *slot_mapping, const int64_t *positions,
                    const float *cos_sin_cache, int64_t max_pos, int32_t block_size,
                    int32_t record, const kvrec_insert_options *options, kvrec_stream stream) {
  if (k_cache == nullptr) return KVREC_ERR_NULL;
  if (!packed_record(record) || record != k_cache->record) return KVREC_ERR_RECORD;
  if (block_size < 1 || block_size != k_cache->block_size) return KVREC_ERR_BLOCK_SIZE;
  kvrec::CacheGeom g;
  const int rc = check_cache(k_cache, &g);
  if (rc != KVREC_OK) return rc;
  const kvrec_insert_options defaults = {KVREC_ROPE_NEOX, 1, 0.0f, 0};
  const kvrec_insert_options &opt = options != nullptr ? *options : defaults;
  if (opt.rope < KVREC_ROPE_NEOX || opt.rope > KVREC_ROPE_NONE) return KVREC_ERR_OPTION;
  if (opt.compress_ratio < 1 || opt.compress_ratio > kMaxCount) return KVREC_ERR_OPTION;
  if (!(opt.amax_floor >= 0.0f) || !isfinite(opt.amax_floor)) return KVREC_ERR_OPTION;
  if (opt.sanitize_nans != 0 && opt.sanitize_nans != 1) return KVREC_ERR_OPTION;
  if (num_tokens < 0 || num_tokens > kMaxCount) return KVREC_ERR_SIZE;
  if (num_tokens == 0) return KVREC_OK;
  // Positions are read for the rotation and the ratio gate, the table only
  // for the rotation; what is not read is neither checked nor passed on
  // (the rotation-free insert with ratio 1 ignores positions and max_pos).
  const bool needs_positions = opt.rope != KVREC_ROPE_NONE || opt.compress_ratio != 1;
  const bool needs_table = opt.rope != KVREC_ROPE_NONE;
  const int64_t *pos = needs_positions ? positions : nullptr;
  const float *table = needs_table ? cos_sin_cache : nullptr;
  if (kv == nullptr || slot_mapping == nullptr) return KVREC_ERR_NULL;
  if ((needs_positions && pos == nullptr) || (needs_table && table == nullptr))
    return KVREC_ERR_NULL;
  if (pos != nullptr && (max_pos < 1 || max_pos > kMaxPos)) return KVREC_ERR_SIZE;
  if (misaligned(kv, 16) || misaligned(table, 16) || misaligned(slot_mapping, 8) ||
      misaligned(pos, 8))
    return KVREC_ERR_ALIGNMENT;
  kvrec::InsertOptions o;
  o.rope = opt.rope;
  o.sanitize = opt.sanitize_nans != 0;
  o.ratio = static_cast<uint32_t>(opt.compress_ratio);
  division_magic(o.ratio, &o.ratio_magic, &o.ratio_shift);
  memcpy(&o.amax_floor_bits, &opt.amax_floor, sizeof o.amax_floor_bits);
  // Without positions the kernels skip the position checks.
  if (pos == nullptr) max_pos = 1;
  const kvrec::Format format =
      record == KVREC_RECORD_LEGACY ? kvrec::Format::kLegacy : kvrec::Format::kMxfp8;
  const hipError_t err =
      kvrec::launch_insert(kv, num_tokens, g, slot_mapping, pos, table, max_pos, format, o,
                           nullptr, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? KVREC_OK : KVREC_ERR_HIP;
}

int kvrec_insert_full(const void *kv, int64_t num_tokens, const kvrec_cache *k_cache,
                      const int64_t *slot_mapping, const int64_t *positions,
                      const float *cos_sin_cache, int64_t max_pos, int32_t block_size,
                      int32_t record, const float *fp8_scale, kvrec_stream stream) {
  if (k_cache == nullptr) return KVREC_ERR_NULL;
  if (!full_record(record) || record != k_cache->record) return KVREC_ERR_RECORD;
  if (block_size < 1 || block_size != k_cache->block_size) return KVREC_ERR_BLOCK_SIZE;
  kvrec::CacheGeom g;
  const int rc = check_cache(k_cache, &g);
  if (rc != KVREC_OK) return rc;
  // The fp8 cache needs its scale ([KV-only op] 实现拆解 1); a scale given
  // for the bf16 cache would be ignored, so it is refused instead.
  if (record == KVREC_RECORD_FP8 && fp8_scale == nullptr) return KVREC_ERR_NULL;
  if (record == KVREC_RECORD_BF16 && fp8_scale != nullptr) return KVREC_ERR_OPTION;
  if (num_tokens < 0 || num_tokens > kMaxCount) return KVREC_ERR_SIZE;
  if (num_tokens == 0) return KVREC_OK;
  if (kv == nullptr || slot_mapping == nullptr || positions == nullptr ||
      cos_sin_cache == nullptr)
    return KVREC_ERR_NULL;
  if (max_pos < 1 || max_pos > kMaxPos) return KVREC_ERR_SIZE;
  if (misaligned(kv, 16) || misaligned(cos_sin_cache, 16) || misaligned(slot_mapping, 8) ||
      misaligned(positions, 8) || misaligned(fp8_scale, 4))
    return KVREC_ERR_ALIGNMENT;
  kvrec::InsertOptions o;
  o.rope = KVREC_ROPE_NEOX;
  o.sanitize = false;
  o.ratio = 1;
  division_magic(1, &o.ratio_magic, &o.ratio_shift);
  o.amax_floor_bits = 0;
  const kvrec::Format format =
      record == KVREC_RECORD_BF16 ? kvrec::Format::kBf16 : kvrec::Format::kFp8;
  const hipError_t err =
      kvrec::launch_insert(kv, num_tokens, g, slot_mapping, positions, cos_sin_cache, max_pos,
                           format, o, fp8_scale, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? KVREC_OK : KVREC_ERR_HIP;
}

int kvrec_qnorm_rope_insert(const void *q_in, void *q_out, int32_t num_heads, float eps,
                            int32_t apply_q_norm, const void *kv, int64_t num_tokens,
                            const kvrec_cache *k_cache, const int64_t *slot_mapping,
                            const int64_t *positions, const float *cos_sin_cache,
                            int64_t max_pos, int32_t block_size, int32_t record,
                            kvrec_stream stream) {
  if (k_cache == nullptr) return KVREC_ERR_NULL;
  if (!packed_record(record) || record != k_cache->record) return KVREC_ERR_RECORD;
  if (block_size < 1 || block_size != k_cache->block_size) return KVREC_ERR_BLOCK_SIZE;
  kvrec::CacheGeom g;
  const int rc = check_cache(k_cache, &g);
  if (rc != KVREC_OK) return rc;
  if (apply_q_norm != 0 && apply_q_norm != 1) return KVREC_ERR_OPTION;
  if (apply_q_norm == 1 && (!(eps > 0.0f) || !isfinite(eps))) return KVREC_ERR_OPTION;
  if (num_heads < 1 || num_heads > kMaxHeads) return KVREC_ERR_SIZE;
  if (num_tokens < 0 || num_tokens > kMaxCount / num_heads) return KVREC_ERR_SIZE;
  if (num_tokens == 0) return KVREC_OK;
  if (q_in == nullptr || q_out == nullptr || kv == nullptr || slot_mapping == nullptr ||
      positions == nullptr || cos_sin_cache == nullptr)
    return KVREC_ERR_NULL;
  if (max_pos < 1 || max_pos > kMaxPos) return KVREC_ERR_SIZE;
  if (misaligned(q_in, 16) || misaligned(q_out, 16) || misaligned(kv, 16) ||
      misaligned(cos_sin_cache, 16) || misaligned(slot_mapping, 8) || misaligned(positions, 8))
    return KVREC_ERR_ALIGNMENT;
  // q_out is q_in (in place) or a separate buffer; a partial overlap would
  // let one wave read rows another has already written.
  const uintptr_t qi = reinterpret_cast<uintptr_t>(q_in), qo = reinterpret_cast<uintptr_t>(q_out);
  const uintptr_t q_bytes = static_cast<uintptr_t>(num_tokens) * num_heads * KVREC_HEAD_DIM * 2;
  if (qi != qo && qi < qo + q_bytes && qo < qi + q_bytes) return KVREC_ERR_OVERLAP;
  kvrec::QArgs q;
  q.in = q_in;
  q.out = q_out;
  q.heads = num_heads;
  q.eps = apply_q_norm == 1 ? eps : 0.0f;
  q.norm = apply_q_norm == 1;
  const hipError_t err =
      kvrec::launch_qkv(q, kv, num_tokens, g, slot_mapping, positions, cos_sin_cache, max_pos,
                        record == KVREC_RECORD_LEGACY, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? KVREC_OK : KVREC_ERR_HIP;
}

int kvrec_gather(const kvrec_cache *k_cache, const int32_t *token_indices, int64_t num_indices,
                 void *out, kvrec_stream stream) {
  kvrec::CacheGeom g;
  const int rc = check_cache(k_cache, &g);
  if (rc != KVREC_OK) return rc;
  if (!packed_record(k_cache->record)) return KVREC_ERR_RECORD;
  if (num_indices < 0 || num_indices > kMaxCount) return KVREC_ERR_SIZE;
  if (num_indices == 0) return KVREC_OK;
  if (token_indices == nullptr || out == nullptr) return KVREC_ERR_NULL;
  if (misaligned(out, 16) || misaligned(token_indices, 4)) return KVREC_ERR_ALIGNMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t err = k_cache->record == KVREC_RECORD_MXFP8
                             ? kvrec::launch_gather_mxfp8(g, token_indices, num_indices, out, s)
                             : kvrec::launch_gather_legacy(g, token_indices, num_indices, out, s);
  return err == hipSuccess ? KVREC_OK : KVREC_ERR_HIP;
}

int kvrec_expand_candidates(const int32_t *candidate_blocks, int64_t cand_stride,
                            const int32_t *row_ks, int64_t ks_stride, const int32_t *row_ke,
                            int64_t ke_stride, int64_t rows, int32_t num_candidates,
                            int32_t ratio, int32_t sparse_block, int32_t *sparse_indices,
                            int64_t sparse_stride, int32_t *end, int64_t end_stride,
                            kvrec_stream stream) {
  // The page's kernel takes K a power of two, RATIO 1 or 2 and SBK 16 or 8
  // (the block sizes its sparse attention accepts).
  if (num_candidates < 1 || num_candidates > kMaxExpanded ||
      (num_candidates & (num_candidates - 1)) != 0)
    return KVREC_ERR_SIZE;
  if (ratio != 1 && ratio != 2) return KVREC_ERR_OPTION;
  if (sparse_block != 8 && sparse_block != 16) return KVREC_ERR_OPTION;
  const int64_t width = static_cast<int64_t>(num_candidates) * ratio;
  if (width > kMaxExpanded) return KVREC_ERR_SIZE;
  if (rows < 0 || rows > kMaxCount) return KVREC_ERR_SIZE;
  if (cand_stride < num_candidates || sparse_stride < width || ks_stride < 1 ||
      ke_stride < 1 || end_stride < 1)
    return KVREC_ERR_SIZE;
  if (rows == 0) return KVREC_OK;
  if (candidate_blocks == nullptr || row_ks == nullptr || row_ke == nullptr ||
      sparse_indices == nullptr || end == nullptr)
    return KVREC_ERR_NULL;
  if (misaligned(candidate_blocks, 4) || misaligned(row_ks, 4) || misaligned(row_ke, 4) ||
      misaligned(sparse_indices, 4) || misaligned(end, 4))
    return KVREC_ERR_ALIGNMENT;
  kvrec::ExpandArgs x;
  x.cand = candidate_blocks;
  x.cand_stride = cand_stride;
  x.ks = row_ks;
  x.ks_stride = ks_stride;
  x.ke = row_ke;
  x.ke_stride = ke_stride;
  x.rows = rows;
  x.num_candidates = num_candidates;
  x.ratio = ratio;
  x.sparse_block = sparse_block;
  x.sparse = sparse_indices;
  x.sparse_stride = sparse_stride;
  x.end = end;
  x.end_stride = end_stride;
  const hipError_t err = kvrec::launch_expand(x, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? KVREC_OK : KVREC_ERR_HIP;
}

const char *kvrec_status_str(int status) {
  switch (status) {
    case KVREC_OK: return "ok";
    case KVREC_ERR_NULL: return "null pointer";
    case KVREC_ERR_RECORD:
      return "record width is not one this call takes (528/584 packed, 1024/512 non-packed), "
             "or does not match the cache";
    case KVREC_ERR_BLOCK_SIZE:
      return "block_size < 1, does not match the cache, or makes a page of 2^31 bytes or more";
    case KVREC_ERR_PAGE_STRIDE:
      return "page stride is not a multiple of the record's page alignment or is too small";
    case KVREC_ERR_ALIGNMENT: return "pointer not aligned as the ABI requires";
    case KVREC_ERR_SIZE: return "size out of range";
    case KVREC_ERR_HIP: return "HIP launch error";
    case KVREC_ERR_OPTION: return "insert option out of range";
    case KVREC_ERR_OVERLAP: return "output buffer partly overlaps an input";
    default: return "unknown kvrec status";
  }
}

}  // extern "C"
