// kvrec_kernels.hip - gfx950 (MI355X, CDNA4) kernels of the paged KV-record
// codec: fused RoPE + MXFP8 (or legacy) quantise + paged insert, with the
// compressed-KV variants (interleaved or no rotation, ratio gate, amax floor,
// NaN sanitising); the same insert into the non-packed bf16 and fp8 caches;
// the attention write (per-head q RMSNorm + RoPE beside the insert); and the
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
// contraction here and no matrix core is used. One wave64 owns two tokens
// (the lesson of [KV-only op] 实现拆解 5: with no query heads to iterate,
// the launch must give every wave tokens of its own, or it idles most of the
// chip). Each wave issues both tokens' loads before it waits on any, encodes
// both, then stores both: two tokens per wave keep twice the bytes in flight
// of one and halve the waves the dispatcher must launch (about 0.2 ns per
// wave on MI355X, 14.6 us for an empty 65536-wave grid), while three or more
// need enough registers to cut occupancy. Lane l holds latent dims 8l..8l+7:
//   - one 16 B global load per lane reads the 1 KB bf16 row, coalesced;
//   - the 64 RoPE dims 448..511 sit in lanes 56..63, and the NeoX partner of
//     dim 448+i is 480+i, i.e. lane l ^ 4: one ds_swizzle (xor 4) exchanges
//     the raw words;
//   - a 32-dim MXFP8 group is 4 adjacent lanes (a DPP quad), a 64-dim legacy
//     group 8 lanes (quad + half-row mirror): amax needs 2 or 3 DPP steps;
//   - the 8 codes of a lane are one 8 B store, so the wave writes the 512 B
//     data row contiguously; the scale bytes are packed across lanes with DPP
//     (or ds_bpermute) and written as dwords.
// Latency. Every load that depends on nothing (the kv row, the slot, the
// position) is issued at once; only the cos/sin row waits for the position.
// The kv row is loaded before the slot is known, so a skipped token costs one
// wasted 1 KB read but no serialised round trip. The bf16 rows read by the
// insert and written by the gather are non-temporal (touched once); records
// and cos/sin rows go through the caches (the launch configuration below
// gives the measured reasons).
//
// Bit-exactness. Built with -ffp-contract=off (no FMA: the rotation is two
// rounded products and one rounded add/subtract, in that order) and with fp32
// denormals preserved. The encode is v_cvt_scalef32_pk_fp8_f32, which divides
// by the power of two 2^e exactly and rounds once to e4m3fn (nearest even;
// |r| * 2^-e never exceeds 448 because of how e is chosen); the decode is
// v_cvt_scalef32_pk_bf16_fp8, which multiplies by 2^e and rounds once to bf16.
// Both take the group's UE8M0 byte as the exponent field of their scale
// operand, so no separate scaling instruction is needed.
#include "kvrec_launch.h"
#include "kvrec_xcd.h"

namespace kvrec {
namespace {

constexpr int kWave = 64;
// s_waitcnt immediate (gfx9 encoding) that waits for every outstanding vector
// memory operation and nothing else: vmcnt 0, expcnt 7, lgkmcnt 15.
constexpr int kWaitVmcnt0 = 0x0F70;

// DPP controls (gfx9 encoding).
constexpr int kQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kHalfRowMirror = 0x141;  // lane i <-> 7-i within 8 lanes
// ds_swizzle bit-mask mode: and 0x1F, or 0, xor 4 -> partner lane l ^ 4.
constexpr int kSwizzleXor4 = 0x1F | (4 << 10);
constexpr int kRowShl4 = 0x104;        // lane i reads lane i+4 of its 16-lane row
constexpr int kRowShl8 = 0x108;
constexpr int kRowShl12 = 0x10C;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Cache policy of each stream, as a bit mask; a set bit makes that stream
// non-temporal (touched once: do not keep it in L2 / Infinity Cache).
enum : int {
  kNtKv = 1,      // insert: bf16 rows
  kNtTable = 2,   // insert: cos/sin rows
  kNtData = 4,    // insert: record data rows
  kNtScale = 8,   // insert: record scale rows
  kNtRecord = 1,  // gather: record loads
  kNtOut = 2,     // gather: bf16 rows
};

template <bool NT, typename T>
__device__ __forceinline__ T ld(const T *p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <bool NT, typename T>
__device__ __forceinline__ void st(T *p, T v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// Counts (n <= 2^30), slots (< 2^30) and positions (max_pos <= 2^31) are
// validated on the host to fit 32 bits, so the kernels index with 32-bit
// scalar arithmetic.
struct InsertArgs {
  const u32x4 *kv;  // [n, 64] x 16 B (bf16 [n, 512])
  const int64_t *slots;
  const int64_t *positions;
  const f32x4 *cos_sin;  // [max_pos, 16] x 16 B (fp32 [max_pos, 64])
  uint8_t *base;
  int64_t page_stride;
  uint32_t n;
  uint32_t block_size;
  uint32_t total_slots;
  uint32_t div_magic;
  uint32_t div_shift;
  uint32_t max_pos;
};

struct GatherArgs {
  const int32_t *indices;
  u32x4 *out;  // [n, 64] x 16 B (bf16 [n, 512])
  const uint8_t *base;
  int64_t page_stride;
  uint32_t n;
  uint32_t block_size;
  uint32_t total_slots;
  uint32_t div_magic;
  uint32_t div_shift;
};

// Page and offset of a slot (< 2^31) by the host's magic-number division.
struct PageOff {
  uint32_t page;
  uint32_t off;
};

__device__ __forceinline__ PageOff page_of(uint32_t slot, uint32_t bs, uint32_t magic,
                                           uint32_t shift) {
  const uint32_t q = (__umulhi(slot, magic) + slot) >> shift;
  return PageOff{q, slot - q * bs};
}

// v < limit for a 64-bit value read from memory, in 32-bit halves (negative
// values have a non-zero high word).
__device__ __forceinline__ bool below(int64_t v, uint32_t limit) {
  return (static_cast<uint64_t>(v) >> 32) == 0 && static_cast<uint32_t>(v) < limit;
}

__device__ __forceinline__ void unpack_bf16x8(const u32x4 w, float f[8]) {
  f[0] = __uint_as_float(w.x << 16);
  f[1] = __uint_as_float(w.x & 0xFFFF0000u);
  f[2] = __uint_as_float(w.y << 16);
  f[3] = __uint_as_float(w.y & 0xFFFF0000u);
  f[4] = __uint_as_float(w.z << 16);
  f[5] = __uint_as_float(w.z & 0xFFFF0000u);
  f[6] = __uint_as_float(w.w << 16);
  f[7] = __uint_as_float(w.w & 0xFFFF0000u);
}

// bf16 bits nearest to two finite fp32 values, ties to even (lo in the low
// half): one v_cvt_pk_bf16_f32, which rounds in the wave's round-to-nearest-
// even mode and keeps fp32 denormals (the kernels run with them enabled).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

template <int Ctrl>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_mov_dpp(static_cast<int>(v), Ctrl, 0xF, 0xF, true));
}

template <int Ctrl>
__device__ __forceinline__ uint32_t dpp_umax(uint32_t v) {
  return max(v, dpp<Ctrl>(v));
}



__device__ __forceinline__ uint32_t lane_read(uint32_t v, int src_lane) {
  return static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(src_lane << 2, static_cast<int>(v)));
}

// Largest |x| of this lane's 8 values, as fp32 bits (compares as unsigned
// integers because every value is finite and non-negative).
__device__ __forceinline__ uint32_t lane_amax_bits(const float f[8]) {
  float m = fmaxf(fmaxf(fabsf(f[0]), fabsf(f[1])), fabsf(f[2]));
  m = fmaxf(fmaxf(m, fabsf(f[3])), fabsf(f[4]));
  m = fmaxf(fmaxf(m, fabsf(f[5])), fabsf(f[6]));
  return __float_as_uint(fmaxf(m, fabsf(f[7])));
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

// The gfx950 scaled conversions read only the exponent field of their fp32
// scale operand, which is exactly a UE8M0 byte: scale = byte << 23 stands for
// 2^(byte - 127). v_cvt_scalef32_pk_fp8_f32 gives e4m3fn(x / 2^(byte-127))
// rounded to nearest even (the division by a power of two is exact, so this
// is one rounding of the exact r * 2^-e); v_cvt_scalef32_pk_bf16_fp8 gives
// bf16(e4m3fn(code) * 2^(byte-127)).
__device__ __forceinline__ float e8m0_as_f32(uint32_t byte) { return __uint_as_float(byte << 23); }

// e4m3fn codes of r * 2^-e for 8 values (scale byte = e + 127), byte k = value k.
__device__ __forceinline__ u32x2 encode_e4m3x8(const float f[8], uint32_t scale_byte) {
  const float sc = e8m0_as_f32(scale_byte);
  // The first conversion of each word writes its low half and keeps the high
  // half of `old`, which the second one then overwrites: any old value works.
  const s16x2 any = __builtin_bit_cast(s16x2, sc);
  s16x2 w0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(any, f[0], f[1], sc, false);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w0, f[2], f[3], sc, true);
  s16x2 w1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(any, f[4], f[5], sc, false);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w1, f[6], f[7], sc, true);
  return u32x2{__builtin_bit_cast(uint32_t, w0), __builtin_bit_cast(uint32_t, w1)};
}

// The NeoX table values of a tail lane. Lanes 56..59 hold x1 = dims 448+i
// and lanes 60..63 x2 = dims 480+i, i = 8*(lane & 3) + k, and both lanes of
// a pair (lane, lane ^ 4) need cos = row[i] and sin = row[32 + i]. Each lane
// loads one half of the row's 256 B once (load_table: lanes 56..59 the cos
// values, 60..63 the sin values, 32 B each), and the pair swaps halves by
// ds_swizzle (xor 4). Measured on MI355X against every tail lane loading all
// 64 B it uses (each half twice): 80.2 -> 69.8 us for 262144 MXFP8 tokens on
// clean caches. All lanes must call it (the swizzle needs the whole wave).
__device__ __forceinline__ void neox_table(int lane, const f32x4 h0, const f32x4 h1, float c[8],
                                           float s[8]) {
  const float own[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
  const bool second = (lane & 4) != 0;  // this lane holds x2 and loaded the sin values
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float other = __uint_as_float(static_cast<uint32_t>(
        __builtin_amdgcn_ds_swizzle(static_cast<int>(__float_as_uint(own[k])), kSwizzleXor4)));
    c[k] = second ? other : own[k];
    s[k] = second ? own[k] : other;
  }
}

// Rotate the tail dims held by lanes 56..63 in place (c, s from neox_table).
// All lanes must call it (the swizzle needs the whole wave); lanes < 56 keep
// their values.
//   r1 = x1*c - x2*s,  r2 = x2*c + x1*s  (each operation rounded separately)
//   With kScaled, the values are x * inv (the q side's normalised rows): the
//   partner's raw bf16 values are multiplied by the same inv, exactly as the
//   partner lane scales its own.
template <bool kScaled = false>
__device__ __forceinline__ void rope_tail(float f[8], const u32x4 raw, int lane, const float c[8],
                                          const float s[8], float inv = 1.0f) {
  // Partner lane l ^ 4 by ds_swizzle (bit-mask mode, no VALU issue: two DPP
  // moves per dword would add 8 VALU instructions, which the fp8 cache's
  // division-heavy insert measurably pays for).
  u32x4 pr;
  pr.x = static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(raw.x), kSwizzleXor4));
  pr.y = static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(raw.y), kSwizzleXor4));
  pr.z = static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(raw.z), kSwizzleXor4));
  pr.w = static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(raw.w), kSwizzleXor4));
  if (lane >= 56) {
    float g[8];
    unpack_bf16x8(pr, g);
    if constexpr (kScaled) {
#pragma unroll
      for (int k = 0; k < 8; ++k) g[k] = g[k] * inv;
    }
    const bool second = (lane & 4) != 0;  // this lane holds x2 (dims 480..)
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float own_c = f[k] * c[k];
      const float other_s = g[k] * s[k];
      f[k] = second ? own_c + other_s : own_c - other_s;
    }
  }
}

// Rotation modes: the NeoX half-split pairs (448+i, 480+i) of the insert,
// the neighbour pairs (2p, 2p+1) of the compressed-KV insert ([MXFP8 record]
// 关键源码片段), or none (the K insert without RoPE).
enum : int { kRopeNeox = 0, kRopeInterleaved = 1, kRopeNone = 2 };

// Cache formats of the insert (kvrec::Format).
constexpr int kFmtMxfp8 = static_cast<int>(Format::kMxfp8);
constexpr int kFmtLegacy = static_cast<int>(Format::kLegacy);
constexpr int kFmtBf16 = static_cast<int>(Format::kBf16);
constexpr int kFmtFp8 = static_cast<int>(Format::kFp8);

// Neighbour-pair rotation. Lane l holds pairs 4l..4l+3 (dims 8l..8l+7), so
// no lane exchange is needed. As in the excerpt, the NoPE pairs (lanes < 56)
// go through the same products with (cos, sin) = (1, 0); lane 56+j uses cos
// row[4j..4j+3] (c0) and sin row[32+4j..32+4j+3] (s0).
__device__ __forceinline__ void rope_interleaved(float f[8], int lane, const f32x4 c0,
                                                 const f32x4 s0) {
  const bool tail = lane >= 56;
  const float c[4] = {tail ? c0.x : 1.0f, tail ? c0.y : 1.0f, tail ? c0.z : 1.0f,
                      tail ? c0.w : 1.0f};
  const float s[4] = {tail ? s0.x : 0.0f, tail ? s0.y : 0.0f, tail ? s0.z : 0.0f,
                      tail ? s0.w : 0.0f};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float xe = f[2 * k], xo = f[2 * k + 1];
    const float xec = xe * c[k], xos = xo * s[k], xoc = xo * c[k], xes = xe * s[k];
    f[2 * k] = xec - xos;
    f[2 * k + 1] = xoc + xes;
  }
}

// One token's record, encoded and held in registers until it is stored:
// this lane's 16 B of the row (8 codes in v.x, v.y for the MXFP8 and fp8
// formats and the legacy NoPE lanes; 8 bf16 in v for the bf16 format and the
// legacy tail lanes) and the packed scale bytes of the lanes that store them.
struct Encoded {
  u32x4 v;
  uint32_t w;
};

// Encode one loaded token. `raw` is the lane's 16 B of the bf16 row, c0..s1
// the lane's cos/sin values (lanes 56..63 only).
template <int kFmt, int kRope, bool kSanitize, bool kOptions>
__device__ __forceinline__ Encoded encode(int lane, const u32x4 raw, const f32x4 c0,
                                          const f32x4 c1, const f32x4 s0, const f32x4 s1,
                                          uint32_t amax_floor_bits, float fp8_scale) {
  constexpr bool kLegacy = kFmt == kFmtLegacy;
  float f[8];
  unpack_bf16x8(raw, f);
  if constexpr (kRope == kRopeNeox) {
    float c[8], sn[8];
    neox_table(lane, c0, c1, c, sn);
    rope_tail(f, raw, lane, c, sn);
  }
  if constexpr (kRope == kRopeInterleaved) rope_interleaved(f, lane, c0, s0);
  if constexpr (kSanitize) {
#pragma unroll
    for (int k = 0; k < 8; ++k) f[k] = f[k] == f[k] ? f[k] : 0.0f;  // NaN -> +0
  }
  Encoded e;
  asm("" : "=v"(e.w));  // only the lanes that store scale bytes set it

  if constexpr (kFmt == kFmtBf16) {
    // Non-packed bf16 cache ([KV-only op] 实现拆解 1): the 1 KB row at
    // page + off*1024. The NoPE lanes store their input bits unchanged (the
    // exact bf16 of an exact widening); the tail lanes round the rotation.
    e.v = raw;
    if (lane >= 56) {
      e.v.x = pack_bf16x2(f[0], f[1]);
      e.v.y = pack_bf16x2(f[2], f[3]);
      e.v.z = pack_bf16x2(f[4], f[5]);
      e.v.w = pack_bf16x2(f[6], f[7]);
    }
    return e;
  }
  if constexpr (kFmt == kFmtFp8) {
    // Non-packed fp8 cache with one fp32 per-tensor scale: the 512 B row at
    // page + off*512 holds e4m3fn(r / scale), saturated to +-448, where r /
    // scale is the IEEE fp32 quotient (rounded once); the conversion then
    // runs with a unit scale (UE8M0 byte 127 = 2^0), rounding to nearest even.
    float y[8];
    const float s = fp8_scale;
    if (s >= 0x1p-90f && s <= 0x1p90f) {
      // The scale is uniform, so its reciprocal is formed once (correctly
      // rounded) and each quotient by Markstein's method (P. Markstein, "IA-64
      // and elementary functions", 2000: if rc is 1/s rounded to nearest and q
      // is faithful, q + (a - s q) rc rounded to nearest is the correctly
      // rounded a / s): q0 = a rc, one fused residual correction (faithful),
      // a second (correctly rounded). a is first clamped to +-1024 s: any
      // larger quotient saturates anyway, and the clamp keeps every
      // intermediate finite; the residuals stay exact down to quotients of
      // 2^-11, below which every result encodes as a signed zero. Each
      // correction is written q - (s q - a) rc, which rounds exactly like
      // q + (a - s q) rc (rounding to nearest is symmetric) but keeps the
      // sign of a zero quotient: -0 / s stays -0 with no separate sign fix.
      // Clamps are one v_med3_f32 each: inputs are finite (a precondition)
      // and s is positive and finite, so no operand is NaN. The +-448 clamp
      // is needed: with a unit scale the conversion rounds values up to 464
      // to 448 but writes the NaN code (0x7F / 0xFF) above that (measured on
      // MI355X), where the cache saturates.
      const float rc = __fdiv_rn(1.0f, s);
      const float lim = 1024.0f * s;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float a = __builtin_amdgcn_fmed3f(f[k], -lim, lim);
        float q = a * rc;
        q = fmaf(-fmaf(s, q, -a), rc, q);
        q = fmaf(-fmaf(s, q, -a), rc, q);
        y[k] = __builtin_amdgcn_fmed3f(q, -448.0f, 448.0f);
      }
    } else {
      // An infinite quotient (tiny s) clamps to +-448 like any other.
#pragma unroll
      for (int k = 0; k < 8; ++k)
        y[k] = __builtin_amdgcn_fmed3f(__fdiv_rn(f[k], s), -448.0f, 448.0f);
    }
    const u32x2 c = encode_e4m3x8(y, 127u);
    e.v = u32x4{c.x, c.y, 0u, 0u};
    return e;
  }

  uint32_t amax = lane_amax_bits(f);
  amax = dpp_umax<kQuadXor1>(amax);
  amax = dpp_umax<kQuadXor2>(amax);
  if constexpr (kLegacy) amax = dpp_umax<kHalfRowMirror>(amax);  // 8 lanes = 64 dims
  if constexpr (kOptions) amax = max(amax, amax_floor_bits);  // the compressed-KV floor
  const int ex = scale_exponent(amax);
  const uint32_t b = static_cast<uint32_t>(ex + 127);

  if constexpr (!kLegacy) {
    // MXFP8 record: 512 codes. Scale byte of group g lives in lanes
    // 4g..4g+3; lane 16k gathers groups 4k..4k+3 from lanes 16k, 16k+4,
    // 16k+8, 16k+12 into one dword.
    const u32x2 c = encode_e4m3x8(f, b);
    e.v = u32x4{c.x, c.y, 0u, 0u};
    e.w = b | (dpp<kRowShl4>(b) << 8) | (dpp<kRowShl8>(b) << 16) | (dpp<kRowShl12>(b) << 24);
  } else {
    // Legacy record: 448 codes of dims 0..447 (lanes 0..55), then the 64
    // rotated tail dims as little-endian bf16 (lanes 56..63).
    if (lane < 56) {
      const u32x2 c = encode_e4m3x8(f, b);
      e.v = u32x4{c.x, c.y, 0u, 0u};
    } else {
      e.v.x = pack_bf16x2(f[0], f[1]);
      e.v.y = pack_bf16x2(f[2], f[3]);
      e.v.z = pack_bf16x2(f[4], f[5]);
      e.v.w = pack_bf16x2(f[6], f[7]);
    }
    // Scale byte of group g lives in lanes 8g..8g+7. Lane 0 packs groups
    // 0..3 (lanes 0, 8, 16, 24), lane 32 packs groups 4..6 and the pad byte.
    const uint32_t b1 = lane_read(b, (lane + 8) & 63);
    const uint32_t b2 = lane_read(b, (lane + 16) & 63);
    const uint32_t r3 = lane_read(b, (lane + 24) & 63);
    const uint32_t b3 = lane == 32 ? 0u : r3;
    e.w = b | (b1 << 8) | (b2 << 16) | (b3 << 24);
  }
  return e;
}

// Store an encoded token at its slot ([MXFP8 record] 功能与动机, 实现拆解 4,
// 关键源码片段: each page holds its data rows, then its scale rows).
//   MXFP8, 528 B: 512 codes at page + off*512, 16 scale bytes at
//     page + block_size*512 + off*16.
//   Legacy, 584 B: a 576 B data row (448 codes, then 64 bf16) at
//     page + off*576, an 8 B scale row (7 scales, then a 0 pad byte) at
//     page + block_size*576 + off*8.
//   bf16 / fp8 rows: page + off*1024 / page + off*512, no scale region.
template <int P, int kFmt>
__device__ __forceinline__ void store_record(const InsertArgs &a, int lane, uint32_t slot,
                                             const Encoded &e) {
  const PageOff po = page_of(slot, a.block_size, a.div_magic, a.div_shift);
  const uint32_t off = po.off;
  uint8_t *page = a.base + static_cast<int64_t>(po.page) * a.page_stride;
  constexpr bool nt_data = (P & kNtData) != 0;
  constexpr bool nt_scale = (P & kNtScale) != 0;
  if constexpr (kFmt == kFmtBf16) {
    st<nt_data>(reinterpret_cast<u32x4 *>(page + off * 1024u + lane * 16), e.v);
  } else if constexpr (kFmt == kFmtFp8) {
    st<nt_data>(reinterpret_cast<u32x2 *>(page + off * 512u + lane * 8), u32x2{e.v.x, e.v.y});
  } else if constexpr (kFmt == kFmtMxfp8) {
    st<nt_data>(reinterpret_cast<u32x2 *>(page + off * 512u + lane * 8), u32x2{e.v.x, e.v.y});
    if ((lane & 15) == 0)
      st<nt_scale>(
          reinterpret_cast<uint32_t *>(page + a.block_size * 512u + off * 16u + (lane >> 2)),
          e.w);
  } else {
    uint8_t *row = page + off * 576u;
    if (lane < 56)
      st<nt_data>(reinterpret_cast<u32x2 *>(row + lane * 8), u32x2{e.v.x, e.v.y});
    else
      st<nt_data>(reinterpret_cast<u32x4 *>(row + 448 + (lane - 56) * 16), e.v);
    if ((lane & 31) == 0)
      st<nt_scale>(
          reinterpret_cast<uint32_t *>(page + a.block_size * 576u + off * 8u + (lane >> 3)),
          e.w);
  }
}

template <int P, int kFmt, int kRope, bool kSanitize, bool kOptions>
__device__ __forceinline__ void encode_store(const InsertArgs &a, int lane, const u32x4 raw,
                                             const f32x4 c0, const f32x4 c1, const f32x4 s0,
                                             const f32x4 s1, uint32_t slot,
                                             uint32_t amax_floor_bits, float fp8_scale) {
  store_record<P, kFmt>(
      a, lane, slot,
      encode<kFmt, kRope, kSanitize, kOptions>(lane, raw, c0, c1, s0, s1, amax_floor_bits,
                                               fp8_scale));
}

// Lanes 56..63 read the cos/sin values of table row `row`. NeoX: lane 56+j
// (j < 4) loads cos[8j .. 8j+7] and lane 60+j loads sin[8j .. 8j+7] into c0,
// c1 (neox_table then swaps halves within the pair; s0, s1 stay unused).
// Interleaved: lane 56+j takes cos[4j .. 4j+3] (c0) and sin[4j .. 4j+3]
// (s0). Other lanes load nothing.
template <int P, int kRope>
__device__ __forceinline__ void load_table(const f32x4 *cos_sin, uint32_t row, int lane,
                                           f32x4 &c0, f32x4 &c1, f32x4 &s0, f32x4 &s1) {
  if (kRope == kRopeNone || lane < 56) return;
  const f32x4 *tab = cos_sin + static_cast<uint64_t>(row) * 16;
  constexpr bool nt = (P & kNtTable) != 0;
  if constexpr (kRope == kRopeNeox) {
    // float4 index of cos[8*(lane&3)] (lanes 56..59) or sin[8*(lane&3)]
    const int q = 2 * (lane & 3) + ((lane & 4) ? 8 : 0);
    c0 = ld<nt>(tab + q);
    c1 = ld<nt>(tab + q + 1);
  } else {
    c0 = ld<nt>(tab + (lane - 56));      // cos of pairs 4j..4j+3
    s0 = ld<nt>(tab + 8 + (lane - 56));  // sin of the same pairs
  }
}

// Insert: wave w of block b handles tokens T*(W*b + w) .. +T-1. For all of
// them it first issues the loads that depend on nothing (kv rows, slots,
// positions), then the cos/sin rows (which need the positions), and only
// then encodes and stores. A token whose slot is negative (or out of range)
// or whose position is out of range is skipped.
// Kernel arguments are plain scalars, ordered so that the ones every wave
// needs first (count, block numbering, input pointers) come first: gfx950
// preloads the leading kernel arguments into SGPRs at wave launch, which
// saves each wave a dependent kernarg load before its first memory request.
// kOptions = false is the plain insert (NeoX, ratio 1, no floor, positions
// present); its code carries none of the option checks below.
// One wave's share of the insert: tokens t0 .. t0+T-1 (t0 < n), ratio 1
// (the compressed-KV gate runs in insert_group_kernel).
template <int P, int T, int kFmt, int kRope, bool kSanitize, bool kOptions>
__device__ __forceinline__ void insert_wave(const InsertArgs &a, uint32_t t0, int lane,
                                            uint32_t amax_floor_bits, const float *fp8_scale) {
  // No positions: only the rotation-free insert (host-checked).
  const bool has_pos = !kOptions || a.positions != nullptr;
  u32x4 raw[T];
  int64_t sl[T], ps[T];
#pragma unroll
  for (int k = 0; k < T; ++k) {
    // A token past the end reloads the last one and is then skipped: the
    // loads stay unconditional, so no loaded register is copied through a
    // branch (a copy would wait for the load before the next is issued).
    const uint32_t t = (T == 1 || t0 + k < a.n) ? t0 + k : a.n - 1;
    raw[k] = ld<(P & kNtKv) != 0>(a.kv + static_cast<uint64_t>(t) * kWave + lane);
    sl[k] = a.slots[t];
    ps[k] = has_pos ? a.positions[t] : 0;
  }
  // All three loads are issued before anything waits on the slot or position.
  __builtin_amdgcn_sched_barrier(0);
  // The page geometry comes in kernel arguments past the ones gfx950 preloads
  // into SGPRs. Reading them here issues their loads beside the slot and
  // position loads, so they arrive with the same wait instead of costing a
  // round trip just before the store.
  asm volatile("" ::"s"(a.block_size), "s"(a.div_magic), "s"(a.div_shift), "s"(a.page_stride),
               "s"(a.base));
  // The fp8 cache's per-tensor scale (one uniform load per wave) is needed
  // only at the encode: it is read after the token's loads are in flight.
  float scale = 1.0f;
  if constexpr (kFmt == kFmtFp8) scale = *fp8_scale;
  uint32_t slot[T], row[T];
  bool ok[T];
#pragma unroll
  for (int k = 0; k < T; ++k) {
    // Bitwise, not short-circuit: a branch here would let the compiler sink
    // a position load behind the wait for the slot.
    ok[k] = static_cast<bool>(static_cast<unsigned>(T == 1 || t0 + k < a.n) &
                              static_cast<unsigned>(below(sl[k], a.total_slots)) &
                              static_cast<unsigned>(!has_pos || below(ps[k], a.max_pos)));
    slot[k] = static_cast<uint32_t>(sl[k]);
    row[k] = static_cast<uint32_t>(ps[k]);
  }
  // The kv row is used only on the encode path; left to itself the compiler
  // sinks its load there, behind the wait for the slot and position. An
  // empty asm reading it on the skip path too keeps the load at the top, in
  // flight together with the slot and position loads.
#pragma unroll
  for (int k = 0; k < T; ++k)
    if (!ok[k]) asm volatile("" ::"v"(raw[k]));
  // Only lanes 56..63 read (and later use) the cos/sin values. The empty asm
  // statements give the registers an unset value in the other lanes, so the
  // compiler does not spend moves per token zero-filling them.
  f32x4 c0[T], c1[T], s0[T], s1[T];
#pragma unroll
  for (int k = 0; k < T; ++k) {
    asm("" : "=v"(c0[k]), "=v"(c1[k]), "=v"(s0[k]), "=v"(s1[k]));
    if (ok[k]) load_table<P, kRope>(a.cos_sin, row[k], lane, c0[k], c1[k], s0[k], s1[k]);
  }
  // Every load of the wave is needed before the first encode. Waiting for all
  // of them here, in one place every path passes, tells the compiler's wait
  // insertion that nothing is outstanding afterwards; left to itself it put a
  // conservative full wait before the second token's stores, which made them
  // wait for the first token's stores to complete (measured on MI355X, legacy
  // 65536 random tokens: 24.1 -> 23.1 us on clean caches, 21.6 -> 20.1 us
  // back to back).
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  // Every token is encoded before any is stored: a store issued between two
  // encodes would make the second one wait for the store to complete (the
  // wait counter covers loads and stores alike).
  Encoded e[T];
#pragma unroll
  for (int k = 0; k < T; ++k)
    if (ok[k])
      e[k] = encode<kFmt, kRope, kSanitize, kOptions>(lane, raw[k], c0[k], c1[k], s0[k], s1[k],
                                                      amax_floor_bits, scale);
#pragma unroll
  for (int k = 0; k < T; ++k)
    if (ok[k]) store_record<P, kFmt>(a, lane, slot[k], e[k]);
}

template <int P, int W, int T, int kFmt, int kRope, bool kSanitize, bool kOptions>
__global__ __launch_bounds__(W * kWave) void insert_kernel(
    uint32_t n, uint32_t xcd_shift, const u32x4 *kv, const int64_t *slots, const int64_t *positions,
    const f32x4 *cos_sin, uint32_t max_pos, uint32_t total_slots, uint8_t *base,
    int64_t page_stride, uint32_t block_size, uint32_t div_magic, uint32_t div_shift,
    uint32_t amax_floor_bits, const float *fp8_scale) {
  const InsertArgs a{kv,         slots,       positions, cos_sin,   base,    page_stride, n,
                     block_size, total_slots, div_magic, div_shift, max_pos};
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const uint32_t t0 = (xcd_block(xcd_shift) * W + wave) * T;
  if (t0 >= a.n) return;
  insert_wave<P, T, kFmt, kRope, kSanitize, kOptions>(a, t0, lane, amax_floor_bits, fp8_scale);
}

// Sum of a value over the 64 lanes, returned in every lane. Each step adds a
// partner lane's value (a + b == b + a in IEEE arithmetic, so every lane ends
// with the same bits): quad xor 1, quad xor 2, 8-lane mirror, 16-lane mirror,
// then lanes 16 and 32 apart.
constexpr int kRowMirror = 0x140;  // lane i <-> 15-i within 16 lanes

__device__ __forceinline__ float wave_sum(float v) {
  v = v + __uint_as_float(dpp<kQuadXor1>(__float_as_uint(v)));
  v = v + __uint_as_float(dpp<kQuadXor2>(__float_as_uint(v)));
  v = v + __uint_as_float(dpp<kHalfRowMirror>(__float_as_uint(v)));
  v = v + __uint_as_float(dpp<kRowMirror>(__float_as_uint(v)));
  const int lane = threadIdx.x & (kWave - 1);
  v = v + __uint_as_float(lane_read(__float_as_uint(v), lane ^ 16));
  v = v + __uint_as_float(lane_read(__float_as_uint(v), lane ^ 32));
  return v;
}

// q side of the attention write for heads h0 .. h0+HPW-1 (those < heads) of
// token t (the QNorm op of [KV-only op] 实现拆解 1; readings: a weightless
// RMSNorm over the head's 512 dims, then the NeoX rotation of the tail with
// the token's table row). Per head: lane l holds dims 8l..8l+7; the sum of
// squares is formed in fp32 (lane-local products and sums, then wave_sum),
// inv = rsq(sum / 512 + eps) (v_rsq_f32, within 1 ulp), y = x * inv, then the
// rotation and round-to-nearest-even bf16. A token whose position is out of
// range leaves its rows unwritten.
template <int P, int HPW, bool kNorm>
__device__ __forceinline__ void qnorm_rope_wave(const InsertArgs &a, const u32x4 *q_in,
                                                u32x4 *q_out, uint32_t t, uint32_t h0,
                                                uint32_t heads, int lane, float eps) {
  // The position (and then the table row, which needs it) is requested
  // before the q rows: measured on MI355X, issuing the 2 KB of q rows first
  // delayed the table row behind them (193 against 180 us at 4096 x 128).
  const int64_t ps = a.positions[t];
  if (!below(ps, a.max_pos)) return;
  f32x4 c0, c1, s0, s1;
  asm("" : "=v"(c0), "=v"(c1), "=v"(s0), "=v"(s1));
  load_table<P, kRopeNeox>(a.cos_sin, static_cast<uint32_t>(ps), lane, c0, c1, s0, s1);
  const uint64_t row0 = static_cast<uint64_t>(t) * heads + h0;
  u32x4 raw[HPW];
#pragma unroll
  for (int k = 0; k < HPW; ++k)
    if (h0 + k < heads) raw[k] = ld<(P & kNtKv) != 0>(q_in + (row0 + k) * kWave + lane);
  float c[8], sn[8];
  neox_table(lane, c0, c1, c, sn);  // once per token, for every head
#pragma unroll
  for (int k = 0; k < HPW; ++k) {
    if (h0 + k >= heads) break;
    float f[8];
    unpack_bf16x8(raw[k], f);
    float inv = 1.0f;
    if constexpr (kNorm) {
      float ss = f[0] * f[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) ss = ss + f[j] * f[j];
      ss = wave_sum(ss);
      inv = __builtin_amdgcn_rsqf(ss * (1.0f / 512.0f) + eps);
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = f[j] * inv;
    }
    rope_tail<kNorm>(f, raw[k], lane, c, sn, inv);
    u32x4 h;
    h.x = pack_bf16x2(f[0], f[1]);
    h.y = pack_bf16x2(f[2], f[3]);
    h.z = pack_bf16x2(f[4], f[5]);
    h.w = pack_bf16x2(f[6], f[7]);
    q_out[(row0 + k) * kWave + lane] = h;
  }
}

// The attention write: the q side for every (token, head group) and the KV
// insert for every token, in one launch. Waves [0, q_waves) take head group
// w % wpt of token w / wpt; waves [q_waves, q_waves + n) take one token's
// insert each. The arguments a q wave needs come first: they fill exactly the
// 16 dwords gfx950 preloads into SGPRs.
template <int P, int kFmt, int HPW, bool kNorm>
__global__ __launch_bounds__(kWave) void qkv_kernel(
    uint32_t xcd_shift, uint32_t q_waves, uint32_t wpt, uint32_t wpt_magic, uint32_t wpt_shift,
    uint32_t heads, float eps, uint32_t max_pos, const u32x4 *q_in, u32x4 *q_out,
    const int64_t *positions, const f32x4 *cos_sin, uint32_t n, const u32x4 *kv,
    const int64_t *slots, uint32_t total_slots, uint8_t *base, int64_t page_stride,
    uint32_t block_size, uint32_t div_magic, uint32_t div_shift) {
  const InsertArgs a{kv,         slots,       positions, cos_sin,   base,    page_stride, n,
                     block_size, total_slots, div_magic, div_shift, max_pos};
  const int lane = threadIdx.x;
  const uint32_t w = xcd_block(xcd_shift);
  if (w < q_waves) {
    const uint32_t t = (__umulhi(w, wpt_magic) + w) >> wpt_shift;
    qnorm_rope_wave<P, HPW, kNorm>(a, q_in, q_out, t, (w - t * wpt) * HPW, heads, lane, eps);
    return;
  }
  const uint32_t t0 = w - q_waves;
  if (t0 >= a.n) return;
  insert_wave<P, 1, kFmt, kRopeNeox, false, false>(a, t0, lane, 0, nullptr);
}

// Grouped insert: each wave takes a group of `group` (<= 64) consecutive
// tokens. Lane j reads the slot and position of token j of the group in one
// vector load (and, for the compressed-KV insert with a ratio R > 1 of
// [MXFP8 record] 关键源码片段, evaluates the gate); a ballot collects the
// tokens to write, and the wave encodes them two at a time so that their kv
// and table loads are in flight together. Against one wave per token this
// replaces the per-token scalar slot/position round trip (the table row waits
// on it) by one vector load per group, and lets a gated-off token cost only
// its slot and position. The work per written token (and every byte written)
// is that of insert_kernel.
template <int P, int kFmt, int kRope, bool kSanitize, bool kOptions, bool kGate>
__global__ __launch_bounds__(kWave) void insert_group_kernel(
    uint32_t n, uint32_t xcd_shift, const u32x4 *kv, const int64_t *slots, const int64_t *positions,
    const f32x4 *cos_sin, uint32_t max_pos, uint32_t total_slots, uint8_t *base,
    int64_t page_stride, uint32_t block_size, uint32_t div_magic, uint32_t div_shift,
    uint32_t ratio, uint32_t ratio_magic, uint32_t ratio_shift, uint32_t amax_floor_bits,
    uint32_t group, const float *fp8_scale) {
  const InsertArgs a{kv,         slots,       positions, cos_sin,   base,    page_stride, n,
                     block_size, total_slots, div_magic, div_shift, max_pos};
  const int lane = threadIdx.x;
  const uint32_t t0 = xcd_block(xcd_shift) * group;
  if (t0 >= a.n) return;
  float scale = 1.0f;
  if constexpr (kFmt == kFmtFp8) scale = *fp8_scale;

  bool ok = false;
  uint32_t slot = 0, row = 0;
  if (static_cast<uint32_t>(lane) < group && t0 + lane < a.n) {
    const int64_t sl = ld<(P & kNtKv) != 0>(a.slots + t0 + lane);
    const int64_t ps = ld<(P & kNtKv) != 0>(a.positions + t0 + lane);
    ok = below(sl, a.total_slots) && below(ps, a.max_pos);
    slot = static_cast<uint32_t>(sl);
    row = static_cast<uint32_t>(ps);
    if constexpr (kGate) {
      // (pos + 1) % R == 0, rotating with row pos / R * R = pos + 1 - R;
      // pos + 1 <= 2^30, so the magic-number division is exact.
      const uint32_t p1 = row + 1;
      const uint32_t q = (__umulhi(p1, ratio_magic) + p1) >> ratio_shift;
      ok = ok && p1 == q * ratio;
      row = p1 - ratio;
    }
  }
  uint64_t kept = __ballot(ok);
  while (kept != 0) {
    const int k0 = __builtin_ctzll(kept);
    kept &= kept - 1;
    const bool two = kept != 0;
    const int k1 = two ? __builtin_ctzll(kept) : k0;
    if (two) kept &= kept - 1;
    const uint32_t slot0 = __builtin_amdgcn_readlane(slot, k0);
    const uint32_t row0 = __builtin_amdgcn_readlane(row, k0);
    const uint32_t slot1 = __builtin_amdgcn_readlane(slot, k1);
    const uint32_t row1 = __builtin_amdgcn_readlane(row, k1);
    constexpr bool nt_kv = (P & kNtKv) != 0;
    const u32x4 raw0 = ld<nt_kv>(a.kv + static_cast<uint64_t>(t0 + k0) * kWave + lane);
    const u32x4 raw1 = ld<nt_kv>(a.kv + static_cast<uint64_t>(t0 + k1) * kWave + lane);
    f32x4 c0, c1, s0, s1, d0, d1, e0, e1;
    asm("" : "=v"(c0), "=v"(c1), "=v"(s0), "=v"(s1));
    asm("" : "=v"(d0), "=v"(d1), "=v"(e0), "=v"(e1));
    load_table<P, kRope>(a.cos_sin, row0, lane, c0, c1, s0, s1);
    load_table<P, kRope>(a.cos_sin, row1, lane, d0, d1, e0, e1);
    encode_store<P, kFmt, kRope, kSanitize, kOptions>(a, lane, raw0, c0, c1, s0, s1, slot0,
                                                      amax_floor_bits, scale);
    if (two)
      encode_store<P, kFmt, kRope, kSanitize, kOptions>(a, lane, raw1, d0, d1, e0, e1, slot1,
                                                        amax_floor_bits, scale);
  }
}

// bf16 of e4m3fn(code) * 2^(scale_byte - 127) for 8 codes, value k = byte k.
__device__ __forceinline__ u32x4 decode_e4m3x8(const u32x2 codes, uint32_t scale_byte) {
  const float sc = e8m0_as_f32(scale_byte);
  return u32x4{
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.x, sc, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.x, sc, true)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.y, sc, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.y, sc, true))};
}

// Gather: index = page*block_size + offset; a negative (or out-of-range)
// index gives a row of +0 ([FlashMLA]: -1 marks an invalid entry). Each wave
// handles kRows consecutive output rows: all index loads first, then all
// record loads, then the decodes and stores.
template <bool kLegacy, int kRows, int P, int W>
__global__ __launch_bounds__(W * kWave) void gather_kernel(
    uint32_t n, uint32_t xcd_shift, const int32_t *indices, const uint8_t *base, int64_t page_stride,
    u32x4 *out, uint32_t total_slots, uint32_t block_size, uint32_t div_magic,
    uint32_t div_shift) {
  const GatherArgs a{indices, out, base, page_stride, n, block_size, total_slots, div_magic,
                     div_shift};
  constexpr bool NT = (P & kNtRecord) != 0;
  constexpr uint32_t kRowBytes = kLegacy ? 576u : 512u;
  constexpr uint32_t kScaleBytes = kLegacy ? 8u : 16u;
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const uint32_t j0 = (xcd_block(xcd_shift) * W + wave) * kRows;
  if (j0 >= a.n) return;

  int32_t idx[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) idx[r] = (j0 + r < a.n) ? a.indices[j0 + r] : -1;

  // Registers of rows (or lanes) that load nothing are left unset (empty asm)
  // instead of zero-filled: those rows store zeros and never read them.
  u32x2 codes[kRows];
  uint32_t sbyte[kRows];
  u32x4 tail[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    asm("" : "=v"(codes[r]), "=v"(sbyte[r]), "=v"(tail[r]));
    if (static_cast<uint32_t>(idx[r]) < a.total_slots) {  // negative -> huge
      const PageOff po =
          page_of(static_cast<uint32_t>(idx[r]), a.block_size, a.div_magic, a.div_shift);
      const uint32_t off = po.off;
      const uint8_t *page = a.base + static_cast<int64_t>(po.page) * a.page_stride;
      const uint8_t *row = page + off * kRowBytes;
      const uint8_t *scales = page + a.block_size * kRowBytes + off * kScaleBytes;
      if (!kLegacy || lane < 56) {
        codes[r] = ld<NT>(reinterpret_cast<const u32x2 *>(row + lane * 8));
        sbyte[r] = ld<NT>(scales + (kLegacy ? (lane >> 3) : (lane >> 2)));
      } else {
        tail[r] = ld<NT>(reinterpret_cast<const u32x4 *>(row + 448 + (lane - 56) * 16));
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    if (j0 + r >= a.n) break;
    u32x4 o = u32x4{0, 0, 0, 0};
    if (static_cast<uint32_t>(idx[r]) < a.total_slots) {
      if (!kLegacy || lane < 56)
        o = decode_e4m3x8(codes[r], sbyte[r]);
      else
        o = tail[r];
    }
    st<(P & kNtOut) != 0>(a.out + static_cast<uint64_t>(j0 + r) * kWave + lane, o);
  }
}

// Launch configuration, chosen by timing every combination on MI355X, both as
// single launches after the caches were cleaned and as the back-to-back
// insert -> gather step (prefill 262144, legacy 65536, decode 16384 and a
// 131072-row top-k gather). The insert's kv rows are non-temporal (touched
// once) while its records are stored normally: they are read back soon, and
// the partial lines of scattered slots merge in cache; the cos/sin rows are
// cached except for the bf16 cache (insert_policy below). The
// gather's bf16 output is non-temporal: written once, and as large as the
// Infinity Cache, it would otherwise evict the records. One wave per insert
// block, two tokens per wave (single launches on clean caches, kernel
// timestamps: MXFP8 262144 contiguous 86.6 -> 80.4 us, legacy 65536 random
// 25.5 -> 23.7 us, fp8 cache 88.6 -> 79.6 us, bf16 cache 94.7 -> 91.2 us;
// back to back the same or faster; three tokens per wave lose occupancy and
// were slower everywhere); two rows per gather wave, two waves per block.
// Cache policy of the insert per format (measured on MI355X, back to back at
// 262144 tokens): the kv rows non-temporal and the cos/sin rows cached took
// the MXFP8 insert from 84.7 to 80.5 us (legacy 84 -> 80, fp8 102 -> 98, the
// gated ratio-4 insert 26.4 -> 24.4); the bf16 cache, which writes 1 KB per
// token, keeps its cos/sin loads non-temporal (91.5 us against 103).
template <int kFmt>
constexpr int insert_policy() {
  return kFmt == kFmtBf16 ? (kNtKv | kNtTable) : kNtKv;
}
constexpr int kInsertWaves = 1;   // waves per block
constexpr int kInsertTokens = 2;  // tokens per wave
constexpr int kGatherPolicy = kNtOut;
constexpr int kGatherWaves = 2;
// q rows (heads) per wave of the attention write. Measured on MI355X at 4096
// tokens x 128 heads, back to back: 1, 2, 4 and 8 heads per wave took 216,
// 180, 188 and 203 us.
constexpr int kQHeadsPerWave = 2;

// Granlund-Montgomery magic for a divisor d >= 1 (as on the host): for every
// n < 2^31, n / d == (umulhi(n, magic) + n) >> shift.
void division_magic32(uint32_t d, uint32_t *magic, uint32_t *shift) {
  uint32_t l = 0;
  while ((uint64_t{1} << l) < d) ++l;
  *magic = static_cast<uint32_t>(((uint64_t{1} << 32) * ((uint64_t{1} << l) - d)) / d + 1);
  *shift = l;
}
constexpr int kGatherRows = 2;    // rows per wave

template <int P, int W, int T, int kFmt, int kRope, bool kSanitize, bool kOptions>
hipError_t launch_insert_slice(const void *kv, int64_t n, const CacheGeom &g,
                               const int64_t *slots, const int64_t *positions,
                               const float *cos_sin, int64_t max_pos, const InsertOptions &o,
                               const float *fp8_scale, hipStream_t stream) {
  uint32_t xcd_shift = 0;
  const dim3 grid = xcd_grid<W>((n + T - 1) / T, &xcd_shift);
  uint32_t n32 = static_cast<uint32_t>(n), mp = static_cast<uint32_t>(max_pos);
  const u32x4 *kv4 = static_cast<const u32x4 *>(kv);
  const f32x4 *cs4 = reinterpret_cast<const f32x4 *>(cos_sin);
  uint8_t *base = g.base;
  int64_t stride = g.page_stride;
  uint32_t total = g.total_slots, bs = g.block_size, magic = g.div_magic, shift = g.div_shift;
  uint32_t floor_bits = o.amax_floor_bits;
  void *params[] = {&n32,  &xcd_shift, &kv4,  &slots, &positions, &cs4,       &mp,
                    &total, &base,    &stride, &bs,   &magic,     &shift,     &floor_bits,
                    &fp8_scale};
  return hipLaunchKernel(
      reinterpret_cast<const void *>(insert_kernel<P, W, T, kFmt, kRope, kSanitize, kOptions>),
      grid,
      dim3(W * kWave), params, 0, stream);
}

template <int P, int W, int T, int kFmt, int kRope, bool kSanitize, bool kOptions>
hipError_t launch_insert(const void *kv, int64_t n, const CacheGeom &g, const int64_t *slots,
                         const int64_t *positions, const float *cos_sin, int64_t max_pos,
                         const InsertOptions &o, const float *fp8_scale, hipStream_t stream) {
  return sliced(n, kMaxLaunchWaves * T, [&](int64_t s, int64_t m) {
    return launch_insert_slice<P, W, T, kFmt, kRope, kSanitize, kOptions>(
        static_cast<const u32x4 *>(kv) + s * kWave, m, g, slots + s,
        positions != nullptr ? positions + s : nullptr, cos_sin, max_pos, o, fp8_scale, stream);
  });
}

// Tokens per wave of the gated insert (ratio R > 1): about two kept tokens
// per group, i.e. one round of loads per wave (measured on MI355X at the
// 262144-token prefill shape: groups of R, 2R, 4R and 8R tokens took 33.6,
// 26.5, 27.8 and 30.0 us at R = 4).
uint32_t gated_group(uint32_t ratio) { return ratio >= 32 ? 64u : 2u * ratio; }

template <int kFmt, int kRope, bool kSanitize, bool kOptions, bool kGate>
hipError_t launch_insert_group_slice(const void *kv, int64_t n, const CacheGeom &g,
                                     const int64_t *slots, const int64_t *positions,
                                     const float *cos_sin, int64_t max_pos,
                                     const InsertOptions &o, uint32_t group,
                                     const float *fp8_scale, hipStream_t stream) {
  uint32_t xcd_shift = 0;
  const dim3 grid = xcd_grid<1>((n + group - 1) / group, &xcd_shift);
  uint32_t n32 = static_cast<uint32_t>(n), mp = static_cast<uint32_t>(max_pos);
  const u32x4 *kv4 = static_cast<const u32x4 *>(kv);
  const f32x4 *cs4 = reinterpret_cast<const f32x4 *>(cos_sin);
  uint8_t *base = g.base;
  int64_t stride = g.page_stride;
  uint32_t total = g.total_slots, bs = g.block_size, magic = g.div_magic, shift = g.div_shift;
  uint32_t ratio = o.ratio, rmagic = o.ratio_magic, rshift = o.ratio_shift;
  uint32_t floor_bits = o.amax_floor_bits;
  void *params[] = {&n32,  &xcd_shift, &kv4,  &slots, &positions, &cs4,   &mp,
                    &total, &base,    &stride, &bs,   &magic,     &shift, &ratio,
                    &rmagic, &rshift, &floor_bits, &group, &fp8_scale};
  return hipLaunchKernel(
      reinterpret_cast<const void *>(
          insert_group_kernel<insert_policy<kFmt>(), kFmt, kRope, kSanitize, kOptions, kGate>),
      grid, dim3(kWave), params, 0, stream);
}

template <int kFmt, int kRope, bool kSanitize, bool kOptions, bool kGate>
hipError_t launch_insert_group(const void *kv, int64_t n, const CacheGeom &g,
                               const int64_t *slots, const int64_t *positions,
                               const float *cos_sin, int64_t max_pos, const InsertOptions &o,
                               uint32_t group, const float *fp8_scale, hipStream_t stream) {
  return sliced(n, kMaxLaunchWaves * group, [&](int64_t s, int64_t m) {
    return launch_insert_group_slice<kFmt, kRope, kSanitize, kOptions, kGate>(
        static_cast<const u32x4 *>(kv) + s * kWave, m, g, slots + s, positions + s, cos_sin,
        max_pos, o, group, fp8_scale, stream);
  });
}

template <int kFmt, int kRope, bool kSanitize, bool kOptions = true>
hipError_t launch_insert_tuned(const void *kv, int64_t n, const CacheGeom &g,
                               const int64_t *slots, const int64_t *positions,
                               const float *cos_sin, int64_t max_pos, const InsertOptions &o,
                               const float *fp8_scale, hipStream_t stream) {
  return launch_insert<insert_policy<kFmt>(), kInsertWaves, kInsertTokens, kFmt, kRope, kSanitize,
                       kOptions>(kv, n, g, slots, positions, cos_sin, max_pos, o, fp8_scale,
                                 stream);
}

template <bool kLegacy, int R, int P, int W>
hipError_t launch_gather_slice(const CacheGeom &g, const int32_t *indices, int64_t n, void *out,
                               hipStream_t stream) {
  uint32_t xcd_shift = 0;
  const dim3 grid = xcd_grid<W>((n + R - 1) / R, &xcd_shift);
  uint32_t n32 = static_cast<uint32_t>(n);
  const uint8_t *base = g.base;
  int64_t stride = g.page_stride;
  u32x4 *out4 = static_cast<u32x4 *>(out);
  uint32_t total = g.total_slots, bs = g.block_size, magic = g.div_magic, shift = g.div_shift;
  void *params[] = {&n32, &xcd_shift, &indices, &base, &stride, &out4, &total, &bs, &magic, &shift};
  return hipLaunchKernel(reinterpret_cast<const void *>(gather_kernel<kLegacy, R, P, W>), grid,
                         dim3(W * kWave), params, 0, stream);
}

template <bool kLegacy, int R, int P, int W>
hipError_t launch_gather(const CacheGeom &g, const int32_t *indices, int64_t n, void *out,
                         hipStream_t stream) {
  return sliced(n, kMaxLaunchWaves * R, [&](int64_t s, int64_t m) {
    return launch_gather_slice<kLegacy, R, P, W>(g, indices + s, m,
                                                 static_cast<u32x4 *>(out) + s * kWave, stream);
  });
}

template <int kFmt, bool kNorm>
hipError_t launch_qkv_slice(const QArgs &q, const void *kv, int64_t n, const CacheGeom &g,
                            const int64_t *slots, const int64_t *positions, const float *cos_sin,
                            int64_t max_pos, hipStream_t stream) {
  uint32_t wpt = static_cast<uint32_t>((q.heads + kQHeadsPerWave - 1) / kQHeadsPerWave);
  uint32_t q_waves = static_cast<uint32_t>(n) * wpt;
  uint32_t xcd_shift = 0;
  const dim3 grid = xcd_grid<1>(static_cast<int64_t>(q_waves) + n, &xcd_shift);
  uint32_t n32 = static_cast<uint32_t>(n), mp = static_cast<uint32_t>(max_pos);
  const u32x4 *kv4 = static_cast<const u32x4 *>(kv);
  const f32x4 *cs4 = reinterpret_cast<const f32x4 *>(cos_sin);
  uint8_t *base = g.base;
  int64_t stride = g.page_stride;
  uint32_t total = g.total_slots, bs = g.block_size, magic = g.div_magic, shift = g.div_shift;
  const u32x4 *qi = static_cast<const u32x4 *>(q.in);
  u32x4 *qo = static_cast<u32x4 *>(q.out);
  uint32_t heads = static_cast<uint32_t>(q.heads);
  uint32_t wmagic = 0, wshift = 0;
  division_magic32(wpt, &wmagic, &wshift);
  float eps = q.eps;
  void *params[] = {&xcd_shift, &q_waves, &wpt,  &wmagic, &wshift, &heads, &eps,
                    &mp,      &qi,      &qo,   &positions, &cs4,  &n32,  &kv4,
                    &slots,   &total,   &base, &stride,    &bs,   &magic, &shift};
  return hipLaunchKernel(
      reinterpret_cast<const void *>(
          qkv_kernel<insert_policy<kFmt>(), kFmt, kQHeadsPerWave, kNorm>),
      grid, dim3(kWave), params, 0, stream);
}

// ceil(heads / 2) q waves and one insert wave per token.
template <int kFmt, bool kNorm>
hipError_t launch_qkv_t(const QArgs &q, const void *kv, int64_t n, const CacheGeom &g,
                        const int64_t *slots, const int64_t *positions, const float *cos_sin,
                        int64_t max_pos, hipStream_t stream) {
  const int64_t waves_per_token = (q.heads + kQHeadsPerWave - 1) / kQHeadsPerWave + 1;
  const int64_t row = q.heads * kWave;  // 16 B units of one token's q rows
  return sliced(n, kMaxLaunchWaves / waves_per_token, [&](int64_t s, int64_t m) {
    QArgs qs = q;
    qs.in = static_cast<const u32x4 *>(q.in) + s * row;
    qs.out = static_cast<u32x4 *>(q.out) + s * row;
    return launch_qkv_slice<kFmt, kNorm>(qs, static_cast<const u32x4 *>(kv) + s * kWave, m, g,
                                         slots + s, positions + s, cos_sin, max_pos, stream);
  });
}

}  // namespace

hipError_t launch_qkv(const QArgs &q, const void *kv, int64_t n, const CacheGeom &g,
                      const int64_t *slots, const int64_t *positions, const float *cos_sin,
                      int64_t max_pos, bool legacy, hipStream_t stream) {
  if (legacy)
    return q.norm ? launch_qkv_t<kFmtLegacy, true>(q, kv, n, g, slots, positions, cos_sin,
                                                   max_pos, stream)
                  : launch_qkv_t<kFmtLegacy, false>(q, kv, n, g, slots, positions, cos_sin,
                                                    max_pos, stream);
  return q.norm ? launch_qkv_t<kFmtMxfp8, true>(q, kv, n, g, slots, positions, cos_sin, max_pos,
                                                stream)
                : launch_qkv_t<kFmtMxfp8, false>(q, kv, n, g, slots, positions, cos_sin, max_pos,
                                                 stream);
}

hipError_t launch_insert(const void *kv, int64_t n, const CacheGeom &g, const int64_t *slots,
                         const int64_t *positions, const float *cos_sin, int64_t max_pos,
                         Format format, const InsertOptions &o, const float *fp8_scale,
                         hipStream_t stream) {
  // The plain insert has its own instantiation per format; the options
  // (packed formats only) get one per (record, rotation, sanitise), with
  // ratio and floor as uniform runtime values.
  const bool plain = o.rope == kRopeNeox && !o.sanitize && o.ratio == 1 &&
                     o.amax_floor_bits == 0 && positions != nullptr;
#define KVREC_PLAIN(F)                                                                        \
  if (plain && format == static_cast<Format>(F))                                              \
    return launch_insert_tuned<F, kRopeNeox, false, false>(kv, n, g, slots, positions, cos_sin, \
                                                         max_pos, o, fp8_scale, stream);
  KVREC_PLAIN(kFmtMxfp8)
  KVREC_PLAIN(kFmtLegacy)
  KVREC_PLAIN(kFmtBf16)
  KVREC_PLAIN(kFmtFp8)
#undef KVREC_PLAIN
  if (format != Format::kMxfp8 && format != Format::kLegacy) return hipErrorInvalidValue;
  const bool legacy = format == Format::kLegacy;
  // Ratio R > 1: the gated group kernel. Ratio 1: the plain insert's
  // kernel shape with the options (measured on MI355X at 262144 tokens, the
  // gated group kernel without its gate took 89-91 us for NeoX + sanitise
  // against 81 us for one wave per token).
#define KVREC_INSERT(L, R, S)                                                                   \
  if (legacy == (L == kFmtLegacy) && o.rope == R && o.sanitize == S) {                          \
    if (o.ratio > 1)                                                                            \
      return launch_insert_group<L, R, S, true, true>(kv, n, g, slots, positions, cos_sin,      \
                                                      max_pos, o, gated_group(o.ratio),         \
                                                      nullptr, stream);                         \
    return launch_insert_tuned<L, R, S>(kv, n, g, slots, positions, cos_sin, max_pos, o,        \
                                        nullptr, stream);                                       \
  }
#define KVREC_INSERT_R(L, R) KVREC_INSERT(L, R, false) KVREC_INSERT(L, R, true)
#define KVREC_INSERT_L(L) \
  KVREC_INSERT_R(L, kRopeNeox) KVREC_INSERT_R(L, kRopeInterleaved) KVREC_INSERT_R(L, kRopeNone)
  KVREC_INSERT_L(kFmtMxfp8)
  KVREC_INSERT_L(kFmtLegacy)
#undef KVREC_INSERT_L
#undef KVREC_INSERT_R
#undef KVREC_INSERT
  return hipErrorInvalidValue;
}

hipError_t launch_gather_mxfp8(const CacheGeom &g, const int32_t *indices, int64_t n, void *out,
                               hipStream_t stream) {
  return launch_gather<false, kGatherRows, kGatherPolicy, kGatherWaves>(g, indices, n, out, stream);
}

hipError_t launch_gather_legacy(const CacheGeom &g, const int32_t *indices, int64_t n, void *out,
                                hipStream_t stream) {
  return launch_gather<true, kGatherRows, kGatherPolicy, kGatherWaves>(g, indices, n, out, stream);
}

}  // namespace kvrec
