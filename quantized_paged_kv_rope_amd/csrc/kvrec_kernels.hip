// kvrec_kernels.hip - gfx950 (MI355X, CDNA4) kernels of the paged KV-record
// codec: fused RoPE + MXFP8 (or legacy) quantise + paged insert, and the
// paged dequantise-and-gather.
//
// Sources (page titles; sections as named on the pages):
//   [MXFP8 record] vLLM PR #56893 report, "[Model][DSv4.1] Store the whole KV
//                  in MXFP8 (FlashMLA V4.1 record)"
//   [KV-only op]   vLLM PR #56441 report, "[Perf][DSpark] Add KV-only context
//                  insertion across V4.1 cache formats"
//   [FlashMLA]     article page "deepseek-ai/FlashMLA" (ssnai.com)
//
// Shape. The path moves ~1.8 KB per token and does ~2 ALU ops per byte, so it
// is bound by HBM bandwidth, not by MFMA or VALU throughput: there is no
// contraction here and no matrix core is used. One wave64 owns one token
// (the lesson of [KV-only op] 实现拆解 5: with no query heads to iterate,
// every wave must have a token of its own, or the launch idles most of the
// chip). Lane l holds latent dims 8l..8l+7:
//   - one 16 B global load per lane reads the 1 KB bf16 row, coalesced;
//   - the 64 RoPE dims 448..511 sit in lanes 56..63, and the NeoX partner of
//     dim 448+i is 480+i, i.e. lane l ^ 4: one ds_swizzle (xor 4) exchanges
//     the raw words;
//   - a 32-dim MXFP8 group is 4 adjacent lanes (a DPP quad), a 64-dim legacy
//     group 8 lanes (quad + half-row mirror): amax needs 2 or 3 DPP steps;
//   - the 8 codes of a lane are one 8 B store; the wave writes the 512 B data
//     row contiguously, and the scale bytes as one 16-lane byte store.
//
// Bit-exactness. Built with -ffp-contract=off (no FMA: the rotation is two
// rounded products and one rounded add/subtract, in that order) and with fp32
// denormals preserved. Scaling by 2^-e uses v_ldexp_f32 (exact, or one
// rounding into the fp32 subnormal range, which e4m3 then rounds to +-0);
// the e4m3fn conversion is v_cvt_pk_fp8_f32 (round to nearest even; inputs
// never exceed 448 in magnitude because of how e is chosen).
#include "kvrec_launch.h"

namespace kvrec {
namespace {

constexpr int kWave = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kBlockThreads = kWave * kWavesPerBlock;

// DPP controls (gfx9 encoding).
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kHalfRowMirror = 0x141;  // lane i <-> 7-i within 8 lanes
// ds_swizzle bit-mask mode: and 0x1F, or 0, xor 4 -> partner lane l ^ 4.
constexpr int kSwizzleXor4 = 0x1F | (4 << 10);

struct InsertArgs {
  const uint4 *kv;  // [n, 64] x 16 B (bf16 [n, 512])
  int64_t n;
  uint8_t *base;
  int64_t page_stride;
  uint32_t block_size;
  uint32_t total_slots;
  const int64_t *slots;
  const int64_t *positions;
  const float4 *cos_sin;  // [max_pos, 16] x 16 B (fp32 [max_pos, 64])
  int64_t max_pos;
};

struct GatherArgs {
  const uint8_t *base;
  int64_t page_stride;
  uint32_t block_size;
  uint32_t total_slots;
  const int32_t *indices;
  int64_t n;
  uint4 *out;  // [n, 64] x 16 B (bf16 [n, 512])
};

__device__ __forceinline__ void unpack_bf16x8(const uint4 &w, float f[8]) {
  f[0] = __uint_as_float(w.x << 16);
  f[1] = __uint_as_float(w.x & 0xFFFF0000u);
  f[2] = __uint_as_float(w.y << 16);
  f[3] = __uint_as_float(w.y & 0xFFFF0000u);
  f[4] = __uint_as_float(w.z << 16);
  f[5] = __uint_as_float(w.z & 0xFFFF0000u);
  f[6] = __uint_as_float(w.w << 16);
  f[7] = __uint_as_float(w.w & 0xFFFF0000u);
}

// bf16 bits nearest to a finite fp32 value, ties to even.
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

template <int Ctrl>
__device__ __forceinline__ uint32_t dpp_umax(uint32_t v) {
  return max(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), Ctrl, 0xF,
                                                                0xF, false)));
}

// Largest |x| of this lane's 8 values, as fp32 bits (compares as unsigned
// integers because every value is finite and non-negative).
__device__ __forceinline__ uint32_t lane_amax_bits(const float f[8]) {
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) m = max(m, __float_as_uint(f[k]) & 0x7FFFFFFFu);
  return m;
}

// UE8M0 exponent of a group ([MXFP8 record] 关键源码片段: ceil(log2(amax/448))):
// the smallest integer e with amax <= 448 * 2^e, clamped to [-127, 127];
// amax == 0 gives 0. With amax = 2^(E-127) * (1 + m/2^23) (normal), 448 * 2^e
// = 1.75 * 2^(e+8), so e = E - 135 when 1 + m/2^23 <= 1.75 (m <= 0x600000) and
// E - 134 otherwise; subnormal and tiny amax fall below the clamp.
__device__ __forceinline__ int scale_exponent(uint32_t amax_bits) {
  if (amax_bits == 0) return 0;
  int e = static_cast<int>(amax_bits >> 23) - 135 + ((amax_bits & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return e < -127 ? -127 : e;  // finite input keeps e <= 120, far below +127
}

// e4m3fn codes of r * 2^-e for 8 values, byte k = value k.
__device__ __forceinline__ uint2 encode_e4m3x8(const float f[8], int e) {
  const int ne = -e;
  float y[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) y[k] = __builtin_amdgcn_ldexpf(f[k], ne);
  int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w0, true);
  int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], w1, true);
  return make_uint2(static_cast<uint32_t>(w0), static_cast<uint32_t>(w1));
}

// Rotate the tail dims held by lanes 56..63 in place. All lanes must call it
// (the swizzle needs the whole wave); lanes < 56 keep their values.
//   lanes 56..59 hold x1 = dims 448+i, lanes 60..63 hold x2 = dims 480+i,
//   i = 8*(lane & 3) + k; cos = row[i], sin = row[32 + i].
//   r1 = x1*c - x2*s,  r2 = x2*c + x1*s  (each operation rounded separately)
__device__ __forceinline__ void rope_tail(float f[8], const uint4 &raw, int lane,
                                          const float4 *row) {
  uint4 pr;
  pr.x = static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(raw.x), kSwizzleXor4));
  pr.y = static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(raw.y), kSwizzleXor4));
  pr.z = static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(raw.z), kSwizzleXor4));
  pr.w = static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(raw.w), kSwizzleXor4));
  if (lane >= 56) {
    float g[8];
    unpack_bf16x8(pr, g);
    const int q = 2 * (lane & 3);  // float4 index of cos[8*(lane&3)]
    const float4 c0 = row[q], c1 = row[q + 1];
    const float4 s0 = row[8 + q], s1 = row[9 + q];
    const float c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    const float s[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    const bool second = (lane & 4) != 0;  // this lane holds x2 (dims 480..)
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float own_c = f[k] * c[k];
      const float other_s = g[k] * s[k];
      f[k] = second ? own_c + other_s : own_c - other_s;
    }
  }
}

// Shared front half of both inserts: returns false if the wave's token is
// skipped; otherwise fills the rotated values and the page/offset.
struct TokenSlot {
  uint8_t *page;
  uint32_t off;
};

__device__ __forceinline__ bool load_rotated(const InsertArgs &a, int64_t t, int lane, float f[8],
                                             TokenSlot &ts) {
  const int64_t slot = a.slots[t];
  if (slot < 0 || slot >= static_cast<int64_t>(a.total_slots)) return false;
  const int64_t pos = a.positions[t];
  if (pos < 0 || pos >= a.max_pos) return false;
  const uint4 raw = a.kv[t * kWave + lane];
  unpack_bf16x8(raw, f);
  rope_tail(f, raw, lane, a.cos_sin + pos * 16);
  const uint32_t s = static_cast<uint32_t>(slot);
  const uint32_t pg = s / a.block_size;
  ts.off = s - pg * a.block_size;
  ts.page = a.base + static_cast<int64_t>(pg) * a.page_stride;
  return true;
}

// MXFP8 record, 528 B: 512 codes at page + off*512, 16 scale bytes at
// page + block_size*512 + off*16 ([MXFP8 record] 功能与动机, 关键源码片段).
__global__ __launch_bounds__(kBlockThreads) void insert_mxfp8_kernel(const InsertArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave;
  if (t >= a.n) return;
  float f[8];
  TokenSlot ts;
  if (!load_rotated(a, t, lane, f, ts)) return;

  uint32_t amax = lane_amax_bits(f);
  amax = dpp_umax<kQuadXor1>(amax);
  amax = dpp_umax<kQuadXor2>(amax);
  const int e = scale_exponent(amax);

  const uint2 codes = encode_e4m3x8(f, e);
  *reinterpret_cast<uint2 *>(ts.page + ts.off * 512u + lane * 8) = codes;
  if ((lane & 3) == 0)
    ts.page[a.block_size * 512u + ts.off * 16u + (lane >> 2)] = static_cast<uint8_t>(e + 127);
}

// Legacy record, 584 B: a 576 B data row (448 codes of dims 0..447, then the
// 64 rotated tail dims as little-endian bf16) at page + off*576, and an 8 B
// scale row (7 scales over 64-dim groups, then a 0 pad byte) at
// page + block_size*576 + off*8 ([MXFP8 record] 功能与动机).
__global__ __launch_bounds__(kBlockThreads) void insert_legacy_kernel(const InsertArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave;
  if (t >= a.n) return;
  float f[8];
  TokenSlot ts;
  if (!load_rotated(a, t, lane, f, ts)) return;

  uint32_t amax = lane_amax_bits(f);
  amax = dpp_umax<kQuadXor1>(amax);
  amax = dpp_umax<kQuadXor2>(amax);
  amax = dpp_umax<kHalfRowMirror>(amax);  // 8 lanes = 64 dims
  const int e = scale_exponent(amax);

  uint8_t *row = ts.page + ts.off * 576u;
  uint8_t *srow = ts.page + a.block_size * 576u + ts.off * 8u;
  if (lane < 56) {
    *reinterpret_cast<uint2 *>(row + lane * 8) = encode_e4m3x8(f, e);
    if ((lane & 7) == 0) srow[lane >> 3] = static_cast<uint8_t>(e + 127);
  } else {
    uint4 h;
    h.x = pack_bf16x2(f[0], f[1]);
    h.y = pack_bf16x2(f[2], f[3]);
    h.z = pack_bf16x2(f[4], f[5]);
    h.w = pack_bf16x2(f[6], f[7]);
    *reinterpret_cast<uint4 *>(row + 448 + (lane - 56) * 16) = h;
    if (lane == 56) srow[7] = 0;
  }
}

// bf16 of e4m3(code) * 2^e for 8 codes (exact products; the rounding only
// matters for e <= -125).
__device__ __forceinline__ uint4 decode_e4m3x8(const uint2 codes, int e) {
  typedef float float2v __attribute__((ext_vector_type(2)));
  const float2v a = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(codes.x), false);
  const float2v b = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(codes.x), true);
  const float2v c = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(codes.y), false);
  const float2v d = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(codes.y), true);
  uint4 o;
  o.x = pack_bf16x2(__builtin_amdgcn_ldexpf(a.x, e), __builtin_amdgcn_ldexpf(a.y, e));
  o.y = pack_bf16x2(__builtin_amdgcn_ldexpf(b.x, e), __builtin_amdgcn_ldexpf(b.y, e));
  o.z = pack_bf16x2(__builtin_amdgcn_ldexpf(c.x, e), __builtin_amdgcn_ldexpf(c.y, e));
  o.w = pack_bf16x2(__builtin_amdgcn_ldexpf(d.x, e), __builtin_amdgcn_ldexpf(d.y, e));
  return o;
}

// Gather: index = page*block_size + offset; a negative (or out-of-range)
// index gives a row of +0 ([FlashMLA]: -1 marks an invalid entry).
__global__ __launch_bounds__(kBlockThreads) void gather_mxfp8_kernel(const GatherArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t j = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave;
  if (j >= a.n) return;
  uint4 *dst = a.out + j * kWave + lane;
  const int32_t idx = a.indices[j];
  if (idx < 0 || static_cast<uint32_t>(idx) >= a.total_slots) {
    *dst = make_uint4(0, 0, 0, 0);
    return;
  }
  const uint32_t s = static_cast<uint32_t>(idx);
  const uint32_t pg = s / a.block_size;
  const uint32_t off = s - pg * a.block_size;
  const uint8_t *page = a.base + static_cast<int64_t>(pg) * a.page_stride;
  const uint2 codes = *reinterpret_cast<const uint2 *>(page + off * 512u + lane * 8);
  const int e = static_cast<int>(page[a.block_size * 512u + off * 16u + (lane >> 2)]) - 127;
  *dst = decode_e4m3x8(codes, e);
}

__global__ __launch_bounds__(kBlockThreads) void gather_legacy_kernel(const GatherArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t j = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave;
  if (j >= a.n) return;
  uint4 *dst = a.out + j * kWave + lane;
  const int32_t idx = a.indices[j];
  if (idx < 0 || static_cast<uint32_t>(idx) >= a.total_slots) {
    *dst = make_uint4(0, 0, 0, 0);
    return;
  }
  const uint32_t s = static_cast<uint32_t>(idx);
  const uint32_t pg = s / a.block_size;
  const uint32_t off = s - pg * a.block_size;
  const uint8_t *page = a.base + static_cast<int64_t>(pg) * a.page_stride;
  const uint8_t *row = page + off * 576u;
  if (lane < 56) {
    const uint2 codes = *reinterpret_cast<const uint2 *>(row + lane * 8);
    const int e = static_cast<int>(page[a.block_size * 576u + off * 8u + (lane >> 3)]) - 127;
    *dst = decode_e4m3x8(codes, e);
  } else {
    *dst = *reinterpret_cast<const uint4 *>(row + 448 + (lane - 56) * 16);
  }
}

inline dim3 grid_for(int64_t n) {
  return dim3(static_cast<unsigned>((n + kWavesPerBlock - 1) / kWavesPerBlock));
}

template <typename Args>
hipError_t launch(void (*kernel)(const Args), const Args &a, int64_t n, hipStream_t stream) {
  void *params[] = {const_cast<Args *>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid_for(n), dim3(kBlockThreads),
                         params, 0, stream);
}

InsertArgs make_insert_args(const void *kv, int64_t n, const CacheGeom &g, const int64_t *slots,
                            const int64_t *positions, const float *cos_sin, int64_t max_pos) {
  InsertArgs a;
  a.kv = static_cast<const uint4 *>(kv);
  a.n = n;
  a.base = g.base;
  a.page_stride = g.page_stride;
  a.block_size = g.block_size;
  a.total_slots = g.total_slots;
  a.slots = slots;
  a.positions = positions;
  a.cos_sin = reinterpret_cast<const float4 *>(cos_sin);
  a.max_pos = max_pos;
  return a;
}

GatherArgs make_gather_args(const CacheGeom &g, const int32_t *indices, int64_t n, void *out) {
  GatherArgs a;
  a.base = g.base;
  a.page_stride = g.page_stride;
  a.block_size = g.block_size;
  a.total_slots = g.total_slots;
  a.indices = indices;
  a.n = n;
  a.out = static_cast<uint4 *>(out);
  return a;
}

}  // namespace

hipError_t launch_insert_mxfp8(const void *kv, int64_t n, const CacheGeom &g, const int64_t *slots,
                               const int64_t *positions, const float *cos_sin, int64_t max_pos,
                               hipStream_t stream) {
  return launch(insert_mxfp8_kernel, make_insert_args(kv, n, g, slots, positions, cos_sin, max_pos),
                n, stream);
}

hipError_t launch_insert_legacy(const void *kv, int64_t n, const CacheGeom &g, const int64_t *slots,
                                const int64_t *positions, const float *cos_sin, int64_t max_pos,
                                hipStream_t stream) {
  return launch(insert_legacy_kernel,
                make_insert_args(kv, n, g, slots, positions, cos_sin, max_pos), n, stream);
}

hipError_t launch_gather_mxfp8(const CacheGeom &g, const int32_t *indices, int64_t n, void *out,
                               hipStream_t stream) {
  return launch(gather_mxfp8_kernel, make_gather_args(g, indices, n, out), n, stream);
}

hipError_t launch_gather_legacy(const CacheGeom &g, const int32_t *indices, int64_t n, void *out,
                                hipStream_t stream) {
  return launch(gather_legacy_kernel, make_gather_args(g, indices, n, out), n, stream);
}

}  // namespace kvrec
