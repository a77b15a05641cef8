/*
 * kvrec_oracle.c - plain CPU reference of the paged KV-record codec.
 *
 * TEST INFRASTRUCTURE: see kvrec_oracle.h. Built with
 *   gcc -O2 -ffp-contract=off -fno-fast-math
 * so every float operation written here is one IEEE-754 binary32 (or
 * binary64) operation rounded to nearest-even, with no fused multiply-add.
 *
 * Structure: each token is processed on its own, in the order the pages
 * state the steps (skip, widen, rotate, per-group amax, scale, encode,
 * store). There is no blocking, vectorisation or reordering.
 *
 * Citation keys are defined in kvrec_oracle.h.
 */
#include "kvrec_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

enum {
  HEAD_DIM = 512,  /* latent width of one token  [MXFP8 record, 功能与动机] */
  ROPE_DIM = 64,   /* rotated tail dims          [KV-only op, 实现拆解 1]  */
  NOPE_DIM = 448,  /* HEAD_DIM - ROPE_DIM                                  */
  HALF_ROPE = 32,
  V41_RECORD = 528,
  V4_RECORD = 584,
};

/* ------------------------------------------------------------------------ */
/* e4m3fn ("float8e4nv" in the excerpt of [MXFP8 record, 关键源码片段]).     */
/* OCP FP8 E4M3: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; no  */
/* infinities; exponent 1111 with mantissa 111 is NaN, so the largest       */
/* finite magnitude is 1.75 * 2^8 = 448.                                    */
/* ------------------------------------------------------------------------ */
double orc_e4m3_value(uint8_t code) {
  int sign = code >> 7;
  int expo = (code >> 3) & 15;
  int mant = code & 7;
  double mag;
  if (expo == 15 && mant == 7) return NAN;
  if (expo == 0)
    mag = ldexp((double)mant, -9);            /* (mant/8) * 2^(1-7)        */
  else
    mag = ldexp((double)(8 + mant), expo - 10); /* (1+mant/8) * 2^(expo-7) */
  return sign ? -mag : mag;
}

/* Round to nearest representable e4m3fn value; on a tie take the value whose
 * code is even (even mantissa); saturate magnitudes >= 448 to 448 (the
 * excerpt clamps to +-448 before the cast [MXFP8 record, 关键源码片段]).
 * The sign bit is copied, so -0 encodes as 0x80. */
uint8_t orc_e4m3_encode(double y) {
  uint8_t sign = signbit(y) ? 0x80 : 0x00;
  double a = fabs(y);
  int lo, hi;
  if (a >= 448.0) return (uint8_t)(sign | 0x7E);
  /* Non-negative codes 0x00..0x7E are ordered by value. Find the bracket
   * value(lo) <= a < value(hi) by bisection. */
  lo = 0x00;
  hi = 0x7E;
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (orc_e4m3_value((uint8_t)mid) <= a)
      lo = mid;
    else
      hi = mid;
  }
  {
    double below = a - orc_e4m3_value((uint8_t)lo); /* exact in binary64 */
    double above = orc_e4m3_value((uint8_t)hi) - a;
    int code;
    if (below < above)
      code = lo;
    else if (above < below)
      code = hi;
    else
      code = (lo % 2 == 0) ? lo : hi;
    return (uint8_t)(sign | code);
  }
}

/* ------------------------------------------------------------------------ */
/* bfloat16: binary32 with the low 16 fraction bits dropped (8 significant  */
/* bits, same exponent range).                                              */
/* ------------------------------------------------------------------------ */
uint16_t orc_bf16_round(double x) {
  uint16_t sign = signbit(x) ? 0x8000 : 0x0000;
  double a = fabs(x);
  int e2;
  int unit;    /* a lies in [2^unit, 2^(unit+1)) */
  int quantum; /* spacing of bf16 values there: 2^quantum */
  double steps, whole, frac, rounded, value;
  float f;
  uint32_t bits;

  if (a == 0.0) return sign;
  (void)frexp(a, &e2); /* a = m * 2^e2, m in [0.5, 1) */
  unit = e2 - 1;
  quantum = (unit < -126 ? -126 : unit) - 7; /* subnormals share 2^-133   */
  steps = ldexp(a, -quantum);                /* exact: power-of-two scale */
  whole = floor(steps);
  frac = steps - whole;
  if (frac > 0.5)
    rounded = whole + 1.0;
  else if (frac < 0.5)
    rounded = whole;
  else
    rounded = (fmod(whole, 2.0) == 0.0) ? whole : whole + 1.0;
  value = ldexp(rounded, quantum);
  if (value >= 0x1p128) return (uint16_t)(sign | 0x7F80); /* +-inf */
  f = (float)value; /* exact: value has <= 8 significant bits */
  memcpy(&bits, &f, sizeof bits);
  return (uint16_t)(sign | (bits >> 16));
}

/* ------------------------------------------------------------------------ */
/* UE8M0 group scale. The excerpt computes ceil(log2(amax / 448)) and stores */
/* it biased by 127 [MXFP8 record, 关键源码片段]. Read as exact real          */
/* arithmetic: the smallest integer e with amax <= 448 * 2^e, so that every  */
/* |x| * 2^-e in the group is <= 448. Clamped to [-127, 127] (byte 0..254).  */
/* amax == 0 (an all-zero group) takes e = 0, byte 127 (no 1e-4 floor).      */
/* ------------------------------------------------------------------------ */
int orc_scale_exponent(float amax) {
  int e;
  if (amax == 0.0f) return 0;
  for (e = -127; e < 127; ++e)
    if ((double)amax <= ldexp(448.0, e)) return e;
  return 127;
}

/* bf16 bits -> binary32 value (exact widening). */
static float widen_bf16(uint16_t h) {
  uint32_t bits = (uint32_t)h << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return f;
}

/* fp32 RoPE of one latent row: dims 0..447 pass through untouched; the tail
 * dims 448..511 are rotated with the NeoX half-split pairing (448+i, 480+i),
 * cos = row[i], sin = row[32+i], products first and then one add/subtract,
 * each a separate binary32 operation:
 *   r[448+i] = (x1*c) - (x2*s),   r[480+i] = (x2*c) + (x1*s).
 * The table layout (32 cos then 32 sin, fp32 [max_pos, 64]) is from
 * [KV-only op, 实现拆解 1]; the product-then-add order is the one in the
 * excerpt of [MXFP8 record, 关键源码片段]. */
static void rope_row(const uint16_t *kv_row, const float *cs_row, float *r) {
  int d, i;
  for (d = 0; d < NOPE_DIM; ++d) r[d] = widen_bf16(kv_row[d]);
  for (i = 0; i < HALF_ROPE; ++i) {
    float x1 = widen_bf16(kv_row[NOPE_DIM + i]);
    float x2 = widen_bf16(kv_row[NOPE_DIM + HALF_ROPE + i]);
    float c = cs_row[i];
    float s = cs_row[HALF_ROPE + i];
    float x1c = x1 * c;
    float x2s = x2 * s;
    float x2c = x2 * c;
    float x1s = x1 * s;
    r[NOPE_DIM + i] = x1c - x2s;
    r[NOPE_DIM + HALF_ROPE + i] = x2c + x1s;
  }
}

/* The compressed-KV insert's rotation ([MXFP8 record] 关键源码片段): the
 * row is viewed as 256 (even, odd) neighbour pairs; pairs 0..223 are the
 * NoPE dims and use (cos, sin) = (1, 0), pairs 224..255 use row[p - 224] and
 * row[32 + p - 224]. Every pair goes through the same two products and one
 * add/subtract, NoPE pairs included (so, e.g., a -0 whose partner is
 * negative comes out +0):
 *   r[2p] = (x[2p] * c) - (x[2p+1] * s),  r[2p+1] = (x[2p+1] * c) + (x[2p] * s). */
static void rope_row_interleaved(const uint16_t *kv_row, const float *cs_row, float *r) {
  int p;
  for (p = 0; p < HEAD_DIM / 2; ++p) {
    float xe = widen_bf16(kv_row[2 * p]);
    float xo = widen_bf16(kv_row[2 * p + 1]);
    int q = p - (NOPE_DIM / 2);
    float c = q >= 0 ? cs_row[q] : 1.0f;
    float s = q >= 0 ? cs_row[HALF_ROPE + q] : 0.0f;
    float xec = xe * c;
    float xos = xo * s;
    float xoc = xo * c;
    float xes = xe * s;
    r[2 * p] = xec - xos;
    r[2 * p + 1] = xoc + xes;
  }
}

static void rotate_row(const uint16_t *kv_row, const float *cs_row, int32_t rope, float *r) {
  int d;
  if (rope == ORC_ROPE_NEOX) {
    rope_row(kv_row, cs_row, r);
  } else if (rope == ORC_ROPE_INTERLEAVED) {
    rope_row_interleaved(kv_row, cs_row, r);
  } else {
    for (d = 0; d < HEAD_DIM; ++d) r[d] = widen_bf16(kv_row[d]);
  }
}

/* Quantise dims [first, first+width) of r as one group: returns the scale
 * byte and writes width e4m3 codes. The element code is the e4m3fn value
 * nearest to the exact product r * 2^-e. The group amax is raised to
 * amax_floor first (the excerpt's floor is 1e-4; 0 leaves it unchanged). */
static uint8_t quantise_group(const float *r, int first, int width, float amax_floor,
                              uint8_t *codes) {
  float amax = 0.0f;
  int d, e;
  for (d = first; d < first + width; ++d)
    if (fabsf(r[d]) > amax) amax = fabsf(r[d]);
  if (amax < amax_floor) amax = amax_floor;
  e = orc_scale_exponent(amax);
  for (d = first; d < first + width; ++d)
    codes[d - first] = orc_e4m3_encode(ldexp((double)r[d], -e));
  return (uint8_t)(e + 127);
}

/* ------------------------------------------------------------------------ */
/* Insert.                                                                  */
/*                                                                          */
/* Token count and slot skip: [KV-only op, 实现拆解 1 and 风险与影响];        */
/* negative slot -> nothing written [MXFP8 record, 关键源码片段].             */
/* Guard (a reading): a slot >= num_blocks*block_size or a position outside  */
/* [0, max_pos) also skips the token (a position only where it is read).    */
/*                                                                          */
/* MXFP8 record (528 B/token) [MXFP8 record, 功能与动机 and 关键源码片段]:    */
/*   page = slot / block_size, off = slot % block_size;                     */
/*   512 codes at page + off*512 (all dims, RoPE dims after rotation);       */
/*   16 UE8M0 bytes (one per 32 dims) at page + block_size*512 + off*16.     */
/*                                                                          */
/* Legacy record (584 B/token) [MXFP8 record, 功能与动机]: 448 NoPE dims as  */
/* e4m3 with 7 UE8M0 scales over 64-dim groups, the 64 rotated RoPE dims as */
/* bf16, 576 B data row then an 8 B scale row (7 scales + 1 pad). Reading:  */
/* data region first (rows of 576 B: codes then little-endian bf16), then   */
/* the scale region (rows of 8 B, pad byte written as 0), as for the MXFP8  */
/* record's data-then-scale page.                                           */
/* ------------------------------------------------------------------------ */
int orc_insert(const uint16_t *kv, int64_t n, uint8_t *cache,
               int64_t num_blocks, int64_t page_stride, int32_t block_size,
               int32_t record, const int64_t *slot_mapping,
               const int64_t *positions, const float *cos_sin_cache,
               int64_t max_pos) {
  orc_insert_options defaults = {ORC_ROPE_NEOX, 1, 0.0f, 0};
  return orc_insert_ex(kv, n, cache, num_blocks, page_stride, block_size, record,
                       slot_mapping, positions, cos_sin_cache, max_pos, &defaults);
}

/* Options beyond the defaults follow the compressed-KV insert of
 * [MXFP8 record] 关键源码片段: a token is written only when
 * (position + 1) % R == 0, and it is rotated with table row position / R * R;
 * the rotated values are NaN-sanitised (NaN -> +0) if asked, before the
 * group amax (raised to the floor) picks the scale. The scale byte cap (254
 * when sanitising, 255 otherwise) cannot bind: e <= 127 already. With no
 * rotation the table is unused and the positions only serve the ratio gate;
 * with ratio 1 both may be NULL (the no-RoPE K insert of [MXFP8 record]
 * 实现拆解 4). */
int orc_insert_ex(const uint16_t *kv, int64_t n, uint8_t *cache, int64_t num_blocks,
                  int64_t page_stride, int32_t block_size, int32_t record,
                  const int64_t *slot_mapping, const int64_t *positions,
                  const float *cos_sin_cache, int64_t max_pos,
                  const orc_insert_options *opts) {
  int64_t t;
  int64_t total_slots = num_blocks * (int64_t)block_size;
  int64_t ratio = opts->compress_ratio;
  if (record != V41_RECORD && record != V4_RECORD) return -1;
  if (ratio < 1 || opts->rope < ORC_ROPE_NEOX || opts->rope > ORC_ROPE_NONE) return -1;
  /* positions (and the table) may be absent only with no rotation and ratio 1 */
  if (positions == NULL && (opts->rope != ORC_ROPE_NONE || ratio != 1)) return -1;
  /* With no rotation and ratio 1 the positions serve nothing (no table row,
   * no gate): they are not read, so no position, in range or not, skips a
   * token. */
  if (opts->rope == ORC_ROPE_NONE && ratio == 1) positions = NULL;

  for (t = 0; t < n; ++t) {
    float r[HEAD_DIM];
    int64_t slot = slot_mapping[t];
    int64_t pos = positions != NULL ? positions[t] : 0;
    int64_t row;
    int64_t page, off;
    uint8_t *pg;
    int g, i, d;

    if (slot < 0 || slot >= total_slots) continue;
    if (positions != NULL) {
      if (pos < 0 || pos >= max_pos) continue;
      if ((pos + 1) % ratio != 0) continue;
    }
    row = pos / ratio * ratio;

    rotate_row(kv + t * HEAD_DIM,
               opts->rope == ORC_ROPE_NONE ? NULL : cos_sin_cache + row * ROPE_DIM, opts->rope,
               r);
    if (opts->sanitize_nans)
      for (d = 0; d < HEAD_DIM; ++d)
        if (r[d] != r[d]) r[d] = 0.0f;

    page = slot / block_size;
    off = slot % block_size;
    pg = cache + page * page_stride;

    if (record == V41_RECORD) {
      uint8_t *data = pg + off * 512;
      uint8_t *scales = pg + (int64_t)block_size * 512 + off * 16;
      for (g = 0; g < 16; ++g)
        scales[g] = quantise_group(r, g * 32, 32, opts->amax_floor, data + g * 32);
    } else {
      uint8_t *data = pg + off * 576;
      uint8_t *scales = pg + (int64_t)block_size * 576 + off * 8;
      for (g = 0; g < 7; ++g)
        scales[g] = quantise_group(r, g * 64, 64, opts->amax_floor, data + g * 64);
      scales[7] = 0;
      for (i = 0; i < ROPE_DIM; ++i) {
        uint16_t h = orc_bf16_round((double)r[NOPE_DIM + i]);
        data[NOPE_DIM + 2 * i] = (uint8_t)(h & 0xFF);
        data[NOPE_DIM + 2 * i + 1] = (uint8_t)(h >> 8);
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Non-packed caches of the KV-only op [KV-only op, 实现拆解 1]: the same    */
/* skip and NeoX rotation, then a plain row of 512 elements per slot at      */
/* page + off * record, with no scale region:                               */
/*   record 1024, bf16 cache: element d is bf16_RNE(r[d]) (dims 0..447 are   */
/*     the input bits unchanged, since r[d] is their exact widening);        */
/*   record 512, fp8 e4m3fn cache with one fp32 per-tensor scale s: element  */
/*     d is the e4m3fn code nearest to the binary32 quotient fl(r[d] / s),   */
/*     saturated to +-448 (a reading: the page requires the fp32 scale but   */
/*     does not print the step; dividing by the scale makes code * s the     */
/*     stored value, and the quotient is formed in fp32, the op's type).     */
/* ------------------------------------------------------------------------ */
int orc_insert_full(const uint16_t *kv, int64_t n, uint8_t *cache, int64_t num_blocks,
                    int64_t page_stride, int32_t block_size, int32_t record,
                    const int64_t *slot_mapping, const int64_t *positions,
                    const float *cos_sin_cache, int64_t max_pos, float fp8_scale) {
  int64_t t;
  int64_t total_slots = num_blocks * (int64_t)block_size;
  if (record != ORC_RECORD_BF16 && record != ORC_RECORD_FP8) return -1;

  for (t = 0; t < n; ++t) {
    float r[HEAD_DIM];
    int64_t slot = slot_mapping[t];
    int64_t pos = positions[t];
    uint8_t *row;
    int d;

    if (slot < 0 || slot >= total_slots) continue;
    if (pos < 0 || pos >= max_pos) continue;
    rope_row(kv + t * HEAD_DIM, cos_sin_cache + pos * ROPE_DIM, r);
    row = cache + (slot / block_size) * page_stride + (slot % block_size) * record;
    if (record == ORC_RECORD_BF16) {
      for (d = 0; d < HEAD_DIM; ++d) {
        uint16_t h = orc_bf16_round((double)r[d]);
        row[2 * d] = (uint8_t)(h & 0xFF);
        row[2 * d + 1] = (uint8_t)(h >> 8);
      }
    } else {
      for (d = 0; d < HEAD_DIM; ++d) {
        float y = r[d] / fp8_scale;
        row[d] = orc_e4m3_encode((double)y);
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* q side of the attention write (the QNorm op whose q_in, q_head_padded,    */
/* eps and apply_q_norm arguments [KV-only op, 实现拆解 1] lists, called in   */
/* [MXFP8 record, 关键源码片段] with padded_heads and eps). The pages name   */
/* the arguments only; the readings taken:                                   */
/*   - q is bf16 [n, heads, 512]; every head of every token is processed      */
/*     (the slot only decides the cache write);                              */
/*   - the norm is an RMSNorm over the head's 512 dims with no weight (none  */
/*     is passed): y = x / sqrt(mean(x^2) + eps); without the norm y = x;    */
/*   - then the same NeoX rotation of dims 448..511 as the KV insert, with   */
/*     the token's table row;                                                */
/*   - each output element is the bf16 nearest to the exact result. It is    */
/*     computed here in binary64 (the sum of squares, the root, the products */
/*     and the rotation), rounded to bf16 once.                             */
/* A token whose position is outside [0, max_pos) leaves its q_out rows      */
/* unwritten.                                                                */
/* ------------------------------------------------------------------------ */
void orc_qnorm_rope(const uint16_t *q_in, int64_t n, int32_t heads, const int64_t *positions,
                    const float *cos_sin_cache, int64_t max_pos, double eps, int32_t apply_norm,
                    uint16_t *q_out) {
  int64_t t;
  int32_t h;
  int d, i;
  for (t = 0; t < n; ++t) {
    int64_t pos = positions[t];
    const float *cs;
    if (pos < 0 || pos >= max_pos) continue;
    cs = cos_sin_cache + pos * ROPE_DIM;
    for (h = 0; h < heads; ++h) {
      const uint16_t *x = q_in + (t * heads + h) * HEAD_DIM;
      uint16_t *out = q_out + (t * heads + h) * HEAD_DIM;
      double y[HEAD_DIM];
      double scale = 1.0;
      if (apply_norm) {
        double sum = 0.0;
        for (d = 0; d < HEAD_DIM; ++d) {
          double v = (double)widen_bf16(x[d]);
          sum += v * v;
        }
        scale = 1.0 / sqrt(sum / HEAD_DIM + eps);
      }
      for (d = 0; d < HEAD_DIM; ++d) y[d] = (double)widen_bf16(x[d]) * scale;
      for (i = 0; i < HALF_ROPE; ++i) {
        double c = cs[i], s = cs[HALF_ROPE + i];
        double y1 = y[NOPE_DIM + i], y2 = y[NOPE_DIM + HALF_ROPE + i];
        y[NOPE_DIM + i] = y1 * c - y2 * s;
        y[NOPE_DIM + HALF_ROPE + i] = y2 * c + y1 * s;
      }
      for (d = 0; d < HEAD_DIM; ++d) out[d] = orc_bf16_round(y[d]);
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Gather (dequantise to bf16). Index = page * block_size + offset; a       */
/* negative index marks an invalid entry [FlashMLA, sparse decode           */
/* integration notes] and yields a row of +0. Reading: an index >=          */
/* num_blocks*block_size is treated the same way.                           */
/* Element: bf16 nearest to e4m3(code) * 2^(scale - 127). The RoPE dims are */
/* returned rotated. Legacy record: dims 448..511 are the stored bf16.      */
/* [MXFP8 record, 实现拆解 4]: one gather parameterised by the fp8 width    */
/* (448 or 512), the group size (64 or 32) and a bf16 tail.                 */
/* ------------------------------------------------------------------------ */
int orc_gather(const uint8_t *cache, int64_t num_blocks, int64_t page_stride,
               int32_t block_size, int32_t record,
               const int32_t *token_indices, int64_t n, uint16_t *out) {
  int64_t j;
  int64_t total_slots = num_blocks * (int64_t)block_size;
  if (record != V41_RECORD && record != V4_RECORD) return -1;

  for (j = 0; j < n; ++j) {
    int64_t idx = token_indices[j];
    uint16_t *row = out + j * HEAD_DIM;
    int64_t page, off;
    const uint8_t *pg;
    int d;

    if (idx < 0 || idx >= total_slots) {
      for (d = 0; d < HEAD_DIM; ++d) row[d] = 0;
      continue;
    }
    page = idx / block_size;
    off = idx % block_size;
    pg = cache + page * page_stride;

    if (record == V41_RECORD) {
      const uint8_t *data = pg + off * 512;
      const uint8_t *scales = pg + (int64_t)block_size * 512 + off * 16;
      for (d = 0; d < HEAD_DIM; ++d) {
        double v = orc_e4m3_value(data[d]) * ldexp(1.0, (int)scales[d / 32] - 127);
        row[d] = orc_bf16_round(v);
      }
    } else {
      const uint8_t *data = pg + off * 576;
      const uint8_t *scales = pg + (int64_t)block_size * 576 + off * 8;
      for (d = 0; d < NOPE_DIM; ++d) {
        double v = orc_e4m3_value(data[d]) * ldexp(1.0, (int)scales[d / 64] - 127);
        row[d] = orc_bf16_round(v);
      }
      for (d = 0; d < ROPE_DIM; ++d)
        row[NOPE_DIM + d] = (uint16_t)(data[NOPE_DIM + 2 * d] |
                                       (data[NOPE_DIM + 2 * d + 1] << 8));
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Candidate-block expansion of the sparse indexer ([Sparse indexer],        */
/* 关键源码片段: the per-row program _expand_candidates_kernel and its        */
/* wrapper candidate_blocks_to_sparse_indices). Per row, in the page's       */
/* order: take the row's K candidate blocks; with RATIO 2 split each         */
/* candidate c into the two sparse blocks 2c and 2c + 1 (in that order);     */
/* keep the blocks b with 0 <= b < ceil(max(ke - ks, 0) / SBK); sort them    */
/* ascending (no de-duplication); add base = ks / SBK; pad the S = K*RATIO   */
/* outputs after the n_valid sorted ones with the last valid block + base   */
/* (base when none is valid); and count the valid sparse token columns,     */
/* end = (n_valid - 1) * SBK + min(max(ke - (last * SBK + ks), 1), SBK), or  */
/* 0 when none is valid (only the last block can be partial). Readings: S = */
/* K * RATIO (the store covers every expanded position); ks >= 0 and ke >= 0 */
/* (so the page's integer division is plain); intermediate values (2c + 1,   */
/* ke - ks + SBK - 1, last * SBK + ks) are exact integers, not wrapped to    */
/* int32 (every stored result fits in int32). This changes results from the  */
/* page's int32 program for rows with ke - ks > 2^31 - SBK only: there its   */
/* ke - ks + SBK - 1 wraps negative and it keeps no block, while this keeps  */
/* the blocks that cover [ks, ke).                                           */
/* ------------------------------------------------------------------------ */
static int compare_int32(const void *a, const void *b) {
  int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
  return (x > y) - (x < y);
}

int orc_expand_candidates(const int32_t *cand, int64_t cand_stride, const int32_t *row_ks,
                          int64_t ks_stride, const int32_t *row_ke, int64_t ke_stride,
                          int64_t rows, int32_t num_candidates, int32_t ratio,
                          int32_t sparse_block, int32_t *sparse, int64_t sparse_stride,
                          int32_t *end, int64_t end_stride) {
  int64_t r;
  int32_t i, j;
  int32_t L = num_candidates * ratio;
  int64_t *blocks;
  int32_t *kept;
  if (num_candidates < 1 || (ratio != 1 && ratio != 2) || sparse_block < 1) return -1;
  blocks = (int64_t *)malloc(sizeof(int64_t) * (size_t)L);
  kept = (int32_t *)malloc(sizeof(int32_t) * (size_t)L);
  if (blocks == NULL || kept == NULL) {
    free(blocks);
    free(kept);
    return -1;
  }
  for (r = 0; r < rows; ++r) {
    const int32_t *c = cand + r * cand_stride;
    int64_t ks = row_ks[r * ks_stride], ke = row_ke[r * ke_stride];
    int64_t kv_len = ke - ks > 0 ? ke - ks : 0;
    int64_t max_block = (kv_len + sparse_block - 1) / sparse_block;
    int64_t base = ks / sparse_block;
    int64_t last = -1, fill, last_start;
    int32_t n_valid = 0, pad;
    int32_t *out = sparse + r * sparse_stride;
    /* expand */
    for (i = 0; i < num_candidates; ++i) {
      if (ratio == 2) {
        blocks[2 * i] = (int64_t)c[i] * 2;
        blocks[2 * i + 1] = (int64_t)c[i] * 2 + 1;
      } else {
        blocks[i] = c[i];
      }
    }
    /* filter */
    for (i = 0; i < L; ++i)
      if (blocks[i] >= 0 && blocks[i] < max_block) {
        kept[n_valid++] = (int32_t)blocks[i];
        if (blocks[i] > last) last = blocks[i];
      }
    /* sort ascending */
    qsort(kept, (size_t)n_valid, sizeof(int32_t), compare_int32);
    /* emit and pad */
    pad = (int32_t)(n_valid > 0 ? last + base : base);
    for (j = 0; j < L; ++j) out[j] = j < n_valid ? (int32_t)(kept[j] + base) : pad;
    last_start = last * sparse_block + ks;
    fill = ke - last_start > 1 ? ke - last_start : 1;
    if (fill > sparse_block) fill = sparse_block;
    end[r * end_stride] = n_valid > 0 ? (int32_t)((n_valid - 1) * (int64_t)sparse_block + fill) : 0;
  }
  free(blocks);
  free(kept);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Batch forms used by the pin tests.                                       */
/* ------------------------------------------------------------------------ */
void orc_e4m3_encode_f32(const float *y, int64_t n, uint8_t *out) {
  int64_t i;
  for (i = 0; i < n; ++i) out[i] = orc_e4m3_encode((double)y[i]);
}

void orc_e4m3_encode_bits(uint32_t first_bits, int64_t n, uint8_t *out) {
  int64_t i;
  for (i = 0; i < n; ++i) {
    uint32_t bits = first_bits + (uint32_t)i;
    float f;
    memcpy(&f, &bits, sizeof f);
    out[i] = orc_e4m3_encode((double)f);
  }
}

void orc_e4m3_value_all(double *out256) {
  int c;
  for (c = 0; c < 256; ++c) out256[c] = orc_e4m3_value((uint8_t)c);
}

void orc_bf16_round_f32(const float *x, int64_t n, uint16_t *out) {
  int64_t i;
  for (i = 0; i < n; ++i) out[i] = orc_bf16_round((double)x[i]);
}

void orc_scale_exponent_f32(const float *amax, int64_t n, int32_t *out) {
  int64_t i;
  for (i = 0; i < n; ++i) out[i] = orc_scale_exponent(amax[i]);
}

void orc_rope_rows_ex(const uint16_t *kv, int64_t n, const int64_t *positions,
                      const float *cos_sin_cache, const orc_insert_options *opts, float *out) {
  int64_t t;
  int d;
  for (t = 0; t < n; ++t) {
    int64_t row = positions[t] / opts->compress_ratio * opts->compress_ratio;
    rotate_row(kv + t * HEAD_DIM, cos_sin_cache + row * ROPE_DIM, opts->rope, out + t * HEAD_DIM);
    if (opts->sanitize_nans)
      for (d = 0; d < HEAD_DIM; ++d)
        if (out[t * HEAD_DIM + d] != out[t * HEAD_DIM + d]) out[t * HEAD_DIM + d] = 0.0f;
  }
}

void orc_rope_rows(const uint16_t *kv, int64_t n, const int64_t *positions,
                   const float *cos_sin_cache, float *out) {
  int64_t t;
  for (t = 0; t < n; ++t)
    rope_row(kv + t * HEAD_DIM, cos_sin_cache + positions[t] * ROPE_DIM,
             out + t * HEAD_DIM);
}
