// kvrec_expand.hip - gfx950 kernel of the sparse indexer's candidate-block
// expansion ([Sparse indexer] 关键源码片段: the per-row program
// _expand_candidates_kernel; page "[DSA] Wire DeepGEMM sparse MQA logits into
// the DeepSeek V4.1 indexer", vLLM PR #56254 report).
//
// Per row: the K candidate blocks (split into 2c, 2c+1 when RATIO is 2) are
// filtered to [0, ceil(max(ke - ks, 0) / SBK)), sorted ascending, anchored at
// ks / SBK and padded with the last kept block; `end` counts the valid sparse
// token columns. Integer work only: the result is exact.
//
// Shape. One wave64 per row. The L = K * RATIO expanded blocks are held in
// registers, E = max(L, 64) / 64 per lane (lane l holds positions
// l*E .. l*E + E-1); positions past L and dropped blocks hold a sentinel
// larger than any kept block. A bitonic network sorts the 64*E keys:
// exchanges at distance < E stay inside a lane, the others go through
// __shfl_xor (ds_bpermute) with lane distance j / E. The kept blocks then
// occupy positions 0 .. n_valid-1 in order, and each lane writes its E
// outputs.
#include "kvrec_launch.h"

namespace kvrec {
namespace {

constexpr int kWave = 64;
constexpr int32_t kSentinel = 0x7FFFFFFF;  // sorts after every kept block

__device__ __forceinline__ int32_t wave_sum_i32(int32_t v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v += __shfl_xor(v, m);
  return v;
}

__device__ __forceinline__ int32_t wave_max_i32(int32_t v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v = max(v, __shfl_xor(v, m));
  return v;
}

template <int E>
__global__ __launch_bounds__(kWave) void expand_kernel(
    const int32_t *cand, int64_t cand_stride, const int32_t *row_ks, int64_t ks_stride,
    const int32_t *row_ke, int64_t ke_stride, uint32_t rows, int32_t num_candidates,
    int32_t ratio, int32_t sbk, int32_t *sparse, int64_t sparse_stride, int32_t *end,
    int64_t end_stride) {
  constexpr int N = kWave * E;
  const uint32_t row = blockIdx.x;
  if (row >= rows) return;
  const int lane = threadIdx.x;
  const int32_t *c = cand + row * cand_stride;
  // Exact integer arithmetic (64-bit where an int32 sum could wrap); every
  // stored value fits in int32. ks and ke are >= 0 (a precondition).
  const int64_t ks = row_ks[row * ks_stride];
  const int64_t ke = row_ke[row * ke_stride];
  const int32_t L = num_candidates * ratio;
  const int64_t kv_len = ke - ks > 0 ? ke - ks : 0;
  const int64_t max_block = (kv_len + sbk - 1) / sbk;
  const int32_t base = static_cast<int32_t>(ks / sbk);

  int32_t a[E];
  int32_t count = 0, last = -1;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int32_t i = lane * E + e;
    int64_t v = -1;
    if (i < L) v = ratio == 2 ? static_cast<int64_t>(c[i >> 1]) * 2 + (i & 1) : c[i];
    const bool keep = i < L && v >= 0 && v < max_block;
    a[e] = keep ? static_cast<int32_t>(v) : kSentinel;
    count += keep ? 1 : 0;
    last = keep ? max(last, static_cast<int32_t>(v)) : last;
  }
  const int32_t n_valid = wave_sum_i32(count);
  last = wave_max_i32(last);

  // Bitonic sort of the N keys, ascending. Position i compares with i ^ j;
  // within each k-sized run the direction is ascending when (i & k) == 0.
#pragma unroll
  for (int k = 2; k <= N; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j < E) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int p = e ^ j;
          if (p > e) {
            const int32_t i = lane * E + e;
            const bool up = (i & k) == 0;
            const int32_t lo = min(a[e], a[p]), hi = max(a[e], a[p]);
            a[e] = up ? lo : hi;
            a[p] = up ? hi : lo;
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int32_t b = __shfl_xor(a[e], j / E);
          const int32_t i = lane * E + e;
          const bool up = (i & k) == 0;
          const bool lower = (i & j) == 0;  // this position is the pair's first
          a[e] = (up == lower) ? min(a[e], b) : max(a[e], b);
        }
      }
    }
  }

  const int32_t pad = n_valid > 0 ? last + base : base;
  int32_t *out = sparse + row * sparse_stride;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int32_t i = lane * E + e;
    if (i < L) out[i] = i < n_valid ? a[e] + base : pad;
  }
  if (lane == 0) {
    const int64_t last_start = static_cast<int64_t>(last) * sbk + ks;
    const int64_t fill = min(max(ke - last_start, int64_t{1}), static_cast<int64_t>(sbk));
    end[row * end_stride] = n_valid > 0 ? (n_valid - 1) * sbk + static_cast<int32_t>(fill) : 0;
  }
}

template <int E>
hipError_t launch_expand_e(const ExpandArgs &x, hipStream_t stream) {
  const int32_t *cand = x.cand, *ks = x.ks, *ke = x.ke;
  int64_t cs = x.cand_stride, kss = x.ks_stride, kes = x.ke_stride, ss = x.sparse_stride,
          es = x.end_stride;
  uint32_t rows = static_cast<uint32_t>(x.rows);
  int32_t k = x.num_candidates, ratio = x.ratio, sbk = x.sparse_block;
  int32_t *sparse = x.sparse, *end = x.end;
  void *params[] = {&cand, &cs,    &ks,  &kss,    &ke, &kes,    &rows,
                    &k,    &ratio, &sbk, &sparse, &ss, &end,    &es};
  return hipLaunchKernel(reinterpret_cast<const void *>(expand_kernel<E>), dim3(rows),
                         dim3(kWave), params, 0, stream);
}

}  // namespace

hipError_t launch_expand(const ExpandArgs &x, hipStream_t stream) {
  const int64_t L = static_cast<int64_t>(x.num_candidates) * x.ratio;
  if (L <= 64) return launch_expand_e<1>(x, stream);
  if (L <= 128) return launch_expand_e<2>(x, stream);
  if (L <= 256) return launch_expand_e<4>(x, stream);
  if (L <= 512) return launch_expand_e<8>(x, stream);
  if (L <= 1024) return launch_expand_e<16>(x, stream);
  return hipErrorInvalidValue;
}

}  // namespace kvrec
