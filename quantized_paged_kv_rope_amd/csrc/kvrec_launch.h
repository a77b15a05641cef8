// kvrec_launch.h - internal interface between the C ABI (kvrec_api.cpp) and
// the gfx950 kernels (kvrec_kernels.hip). Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvrec {

// Waves of one kernel launch, at most. A call with more rows runs as several
// launches on its stream, each over a contiguous slice of the rows (every
// kernel indexes its rows relative to the pointers it is given), so a grid
// never approaches the 2^32 work-items one dispatch can cover.
constexpr int64_t kMaxLaunchWaves = int64_t{1} << 21;

// Geometry of a validated cache (all checks done on the host).
struct CacheGeom {
  uint8_t *base;
  int64_t page_stride;
  uint32_t block_size;
  uint32_t total_slots;  // num_blocks * block_size, <= 2^30
  uint32_t div_magic;    // slot / block_size == (umulhi(slot, div_magic) + slot) >> div_shift
  uint32_t div_shift;    //   for every slot < 2^31
};

// Cache format written by the insert: the packed records (528 B MXFP8,
// 584 B legacy) and the non-packed rows (1024 B bf16, 512 B e4m3fn with a
// per-tensor scale).
enum class Format : int { kMxfp8 = 0, kLegacy = 1, kBf16 = 2, kFp8 = 3 };

// Validated insert options (see kvrec_insert_options in kvrec.h).
struct InsertOptions {
  int rope;                  // 0 NeoX, 1 interleaved, 2 none
  bool sanitize;             // rotated NaN -> +0
  uint32_t ratio;            // compress ratio, >= 1
  uint32_t ratio_magic;      // p / ratio == (umulhi(p, ratio_magic) + p) >> ratio_shift
  uint32_t ratio_shift;      //   for every p < 2^31
  uint32_t amax_floor_bits;  // fp32 bits of the amax floor (0 = none)
};

// fp8_scale (device, one fp32) is read only by Format::kFp8; the options
// apply to the packed formats only (the non-packed ones take the defaults).
hipError_t launch_insert(const void *kv, int64_t n, const CacheGeom &g, const int64_t *slots,
                         const int64_t *positions, const float *cos_sin, int64_t max_pos,
                         Format format, const InsertOptions &o, const float *fp8_scale,
                         hipStream_t stream);
// q side of the attention write: bf16 [n, heads, 512] rows in and out (out
// may be in), normalised with eps when norm is set.
struct QArgs {
  const void *in;
  void *out;
  int64_t heads;
  float eps;
  bool norm;
};

// The attention write: the q side plus the plain insert into a packed cache,
// in one launch.
hipError_t launch_qkv(const QArgs &q, const void *kv, int64_t n, const CacheGeom &g,
                      const int64_t *slots, const int64_t *positions, const float *cos_sin,
                      int64_t max_pos, bool legacy, hipStream_t stream);
// Candidate-block expansion of the sparse indexer (kvrec_expand.hip).
struct ExpandArgs {
  const int32_t *cand;
  int64_t cand_stride;
  const int32_t *ks;
  int64_t ks_stride;
  const int32_t *ke;
  int64_t ke_stride;
  int64_t rows;
  int32_t num_candidates;  // K, a power of two; K * ratio <= 1024
  int32_t ratio;           // 1 or 2
  int32_t sparse_block;    // SBK
  int32_t *sparse;
  int64_t sparse_stride;
  int32_t *end;
  int64_t end_stride;
};

hipError_t launch_expand(const ExpandArgs &x, hipStream_t stream);
hipError_t launch_gather_mxfp8(const CacheGeom &g, const int32_t *indices, int64_t n, void *out,
                               hipStream_t stream);
hipError_t launch_gather_legacy(const CacheGeom &g, const int32_t *indices, int64_t n, void *out,
                                hipStream_t stream);

}  // namespace kvrec
