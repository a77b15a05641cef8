// kvrec_api.cpp - the C ABI declared in include/kvrec.h: argument checks on
// the host, then one kernel launch on the caller's stream.
//
// Checks follow the validation list of the page's KV-only op ([KV-only op]
// 实现拆解 1: dtype/shape/stride/record-width checks at the op's entry, and
// nothing runs on failure), restated for plain pointers: the record width
// selects the kernel, the block size is cross-checked against the cache, the
// page stride must be a multiple of the record's page alignment (512 B for
// the 528 B record, 576 B for the 584 B record: [MXFP8 record] 功能与动机).
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "kvrec.h"
#include "kvrec_launch.h"

namespace {

constexpr int64_t kMaxCount = int64_t{1} << 30;  // rows and slots; keeps grids < 2^31 blocks
constexpr int64_t kMaxPos = int64_t{1} << 31;    // cos/sin rows (a 512 GB table)

bool misaligned(const void *p, uintptr_t align) {
  return (reinterpret_cast<uintptr_t>(p) & (align - 1)) != 0;
}

int64_t record_alignment(int32_t record) { return record == KVREC_RECORD_MXFP8 ? 512 : 576; }

bool known_record(int32_t record) {
  return record == KVREC_RECORD_MXFP8 || record == KVREC_RECORD_LEGACY;
}

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
  if (block_size < 1) return KVREC_ERR_BLOCK_SIZE;
  const int64_t align = record_alignment(record);
  const int64_t raw = static_cast<int64_t>(block_size) * record;
  *page_stride_out = (raw + align - 1) / align * align;
  return KVREC_OK;
}

int kvrec_insert(const void *kv, int64_t num_tokens, const kvrec_cache *k_cache,
                 const int64_t *slot_mapping, const int64_t *positions,
                 const float *cos_sin_cache, int64_t max_pos, int32_t block_size,
                 int32_t record, kvrec_stream stream) {
  if (k_cache == nullptr) return KVREC_ERR_NULL;
  if (!known_record(record) || record != k_cache->record) return KVREC_ERR_RECORD;
  if (block_size < 1 || block_size != k_cache->block_size) return KVREC_ERR_BLOCK_SIZE;
  kvrec::CacheGeom g;
  const int rc = check_cache(k_cache, &g);
  if (rc != KVREC_OK) return rc;
  if (num_tokens < 0 || num_tokens > kMaxCount) return KVREC_ERR_SIZE;
  if (num_tokens == 0) return KVREC_OK;
  if (kv == nullptr || slot_mapping == nullptr || positions == nullptr || cos_sin_cache == nullptr)
    return KVREC_ERR_NULL;
  if (max_pos < 1 || max_pos > kMaxPos) return KVREC_ERR_SIZE;
  if (misaligned(kv, 16) || misaligned(cos_sin_cache, 16) || misaligned(slot_mapping, 8) ||
      misaligned(positions, 8))
    return KVREC_ERR_ALIGNMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t err =
      record == KVREC_RECORD_MXFP8
          ? kvrec::launch_insert_mxfp8(kv, num_tokens, g, slot_mapping, positions, cos_sin_cache,
                                       max_pos, s)
          : kvrec::launch_insert_legacy(kv, num_tokens, g, slot_mapping, positions,
                                        cos_sin_cache, max_pos, s);
  return err == hipSuccess ? KVREC_OK : KVREC_ERR_HIP;
}

int kvrec_gather(const kvrec_cache *k_cache, const int32_t *token_indices, int64_t num_indices,
                 void *out, kvrec_stream stream) {
  kvrec::CacheGeom g;
  const int rc = check_cache(k_cache, &g);
  if (rc != KVREC_OK) return rc;
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

const char *kvrec_status_str(int status) {
  switch (status) {
    case KVREC_OK: return "ok";
    case KVREC_ERR_NULL: return "null pointer";
    case KVREC_ERR_RECORD: return "record width is not 528 or 584, or does not match the cache";
    case KVREC_ERR_BLOCK_SIZE: return "block_size < 1 or does not match the cache";
    case KVREC_ERR_PAGE_STRIDE:
      return "page stride is not a multiple of the record's page alignment or is too small";
    case KVREC_ERR_ALIGNMENT: return "pointer not aligned as the ABI requires";
    case KVREC_ERR_SIZE: return "size out of range";
    case KVREC_ERR_HIP: return "HIP launch error";
    default: return "unknown kvrec status";
  }
}

}  // extern "C"
