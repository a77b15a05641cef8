// kvrec_launch.h - internal interface between the C ABI (kvrec_api.cpp) and
// the gfx950 kernels (kvrec_kernels.hip). Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvrec {

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
hipError_t launch_gather_mxfp8(const CacheGeom &g, const int32_t *indices, int64_t n, void *out,
                               hipStream_t stream);
hipError_t launch_gather_legacy(const CacheGeom &g, const int32_t *indices, int64_t n, void *out,
                                hipStream_t stream);

}  // namespace kvrec
