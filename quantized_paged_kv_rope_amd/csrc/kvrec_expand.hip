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
// Shape. One wave64 per row, two waves per block; each wave has its own LDS
// share and orders only its own LDS accesses, so the two rows of a block may
// take different paths below. The L = K * RATIO expanded blocks are held in
// registers, E = max(L, 64) / 64 per lane (lane l holds positions
// l*E .. l*E + E-1); positions past L and dropped blocks hold a sentinel
// larger than any kept block. The kept count comes from ballots. Two ways to
// order the kept blocks, chosen per row (the choice is uniform in the wave):
//
// - Rank sort, when the row has at most kRankMaxBlocks blocks and its kept
//   blocks are distinct (the candidates of a top-k are): each kept block sets
//   its bit in a bitmap in LDS; a prefix sum of the words' popcounts gives
//   every block its rank, the number of kept blocks below it; each block is
//   written to its rank in an LDS row and read back in order (with RATIO 2
//   the two blocks of a candidate share one bitmap update and one rank). The
//   bitmap's popcount equals the kept count exactly when no block repeats,
//   so a repeated block sends the row to the network below.
// - A bitonic network otherwise: exchanges at distance < E stay inside a
//   lane; the others read the partner lane by DPP (lane distances 1..8),
//   ds_swizzle (16) or ds_bpermute (32), and keep the smaller or larger key
//   by one compare and one select, the direction being a per-stage property
//   of the lane.
//
// Either way the kept blocks end at positions 0 .. n_valid-1 in ascending
// order, and each lane writes its E outputs.
#include "kvrec_launch.h"
#include "kvrec_xcd.h"

namespace kvrec {
namespace {

constexpr int kWave = 64;
constexpr int32_t kSentinel = 0x7FFFFFFF;  // sorts after every kept block

// DPP controls (gfx9 encoding) and the ds_swizzle bit-mask pattern for xor 16.
constexpr int kQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]: lane l ^ 1
constexpr int kQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]: lane l ^ 2
constexpr int kQuadReverse = 0x1B;   // quad_perm [3,2,1,0]: lane l ^ 3
constexpr int kHalfRowMirror = 0x141;  // lane l ^ 7 within 8 lanes
constexpr int kRowRotate8 = 0x128;     // row_ror:8, i.e. lane l ^ 8 within 16 lanes
constexpr int kRowShr1 = 0x111;        // row_shr:n is 0x110 + n: lane l - n within a row
constexpr int kSwizzleXor16 = 0x1F | (16 << 10);

// Rank sort limits: rows of up to 16384 blocks (a 512-word bitmap, at most 8
// words per lane).
constexpr int kRankMaxBlocks = 16384;
constexpr int kRankWords = kRankMaxBlocks / 32;

template <int Ctrl>
__device__ __forceinline__ int32_t dpp(int32_t v) {
  return __builtin_amdgcn_mov_dpp(v, Ctrl, 0xF, 0xF, true);
}

// The value held by lane l ^ D. Distances 1..8 are DPP moves (VALU, no LDS
// round trip): xor 4 = (xor 7) then (xor 3), xor 8 = a rotation of the
// 16-lane row by 8; 16 is a ds_swizzle within 32 lanes, 32 a ds_bpermute.
template <int D>
__device__ __forceinline__ int32_t lane_xor(int32_t v, int32_t addr_xor32) {
  if constexpr (D == 1) return dpp<kQuadXor1>(v);
  else if constexpr (D == 2) return dpp<kQuadXor2>(v);
  else if constexpr (D == 4) return dpp<kQuadReverse>(dpp<kHalfRowMirror>(v));
  else if constexpr (D == 8) return dpp<kRowRotate8>(v);
  else if constexpr (D == 16) return __builtin_amdgcn_ds_swizzle(v, kSwizzleXor16);
  else return __builtin_amdgcn_ds_bpermute(addr_xor32, v);
}

// One stage of the bitonic network at distance J within runs of K keys, for
// keys at positions i = lane * E + e. Position i keeps the smaller key of its
// pair (i, i ^ J) when it is the pair's first and the run ascends
// ((i & K) == 0), or when it is the second and the run descends; otherwise
// the larger.
template <int E, int K, int J>
__device__ __forceinline__ void bitonic_stage(int32_t (&a)[E], int lane, int32_t addr_xor32) {
  if constexpr (J < E) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int p = e ^ J;
      if (p > e) {
        if constexpr (K < E) {
          // direction fixed by e alone
          const int32_t lo = min(a[e], a[p]), hi = max(a[e], a[p]);
          if ((e & K) == 0) {
            a[e] = lo;
            a[p] = hi;
          } else {
            a[e] = hi;
            a[p] = lo;
          }
        } else {
          // direction from the lane: ascending when ((lane * E) & K) == 0
          const bool up = ((lane * E) & K) == 0;
          const bool swap = (a[e] > a[p]) == up;
          const int32_t x = a[e], y = a[p];
          a[e] = swap ? y : x;
          a[p] = swap ? x : y;
        }
      }
    }
  } else {
    // partner in lane l ^ (J / E); keep the larger key when exactly one of
    // "run descends" and "second of the pair" holds.
    const bool keep_max = ((((lane * E) & K) != 0) != (((lane * E) & J) != 0));
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int32_t b = lane_xor<J / E>(a[e], addr_xor32);
      const bool take_b = (a[e] > b) != keep_max;
      a[e] = take_b ? b : a[e];
    }
  }
}

template <int E, int K, int J>
__device__ __forceinline__ void bitonic_merge(int32_t (&a)[E], int lane, int32_t addr_xor32) {
  bitonic_stage<E, K, J>(a, lane, addr_xor32);
  if constexpr (J > 1) bitonic_merge<E, K, J / 2>(a, lane, addr_xor32);
}

template <int E, int K>
__device__ __forceinline__ void bitonic_sort(int32_t (&a)[E], int lane, int32_t addr_xor32) {
  if constexpr (K <= kWave * E) {
    bitonic_merge<E, K, K / 2>(a, lane, addr_xor32);
    bitonic_sort<E, K * 2>(a, lane, addr_xor32);
  }
}

// Exclusive prefix sum of v over the 64 lanes; *total receives the sum over
// all lanes. Inclusive sums within each 16-lane row by four DPP shifts (a
// lane whose source lies before its row adds 0), then each row adds the
// totals of the rows before it.
template <int N>
__device__ __forceinline__ uint32_t row_shr(uint32_t v) {  // 0 where l - N leaves the row
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int32_t>(v), kRowShr1 + N - 1, 0xF, 0xF, false));
}

__device__ __forceinline__ uint32_t wave_exclusive_sum(uint32_t v, int lane, uint32_t *total) {
  uint32_t s = v;
  s += row_shr<1>(s);
  s += row_shr<2>(s);
  s += row_shr<4>(s);
  s += row_shr<8>(s);
  const uint32_t r0 = __builtin_amdgcn_readlane(s, 15), r1 = __builtin_amdgcn_readlane(s, 31),
                 r2 = __builtin_amdgcn_readlane(s, 47), r3 = __builtin_amdgcn_readlane(s, 63);
  *total = r0 + r1 + r2 + r3;
  const uint32_t before = lane < 16 ? 0u : lane < 32 ? r0 : lane < 48 ? r0 + r1 : r0 + r1 + r2;
  return s + before - v;
}

// Orders one wave's LDS accesses across this point: every lane's earlier
// accesses complete before any later one starts (the workgroup-scope fence
// waits for them) and the compiler moves none across it. The waves of a
// block never wait for each other: each owns its row and its share of LDS.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Rank sort of the kept keys of one row into ascending order (positions
// 0 .. n_valid-1 of a[]), for keys in [0, 32 * words) with words <= kRankWords.
// Returns false, leaving a[] as it was, when a key repeats.
//
// kPairs (RATIO 2, E >= 2): a[2m] and a[2m+1] are the blocks 2c and 2c + 1 of
// one candidate c. They share a bitmap word, and 2c + 1 is kept only when 2c
// is, so one update sets both bits and rank(2c + 1) = rank(2c) + 1.
template <int E, bool kPairs>
__device__ __forceinline__ bool rank_sort(int32_t (&a)[E], int lane, uint32_t words,
                                          int32_t n_valid, uint2 *bitmap, int32_t *sorted) {
  // Words [0, 64 q) are used, lane l owning l*q .. l*q + q-1; those past
  // `words` stay zero. The loops over a lane's words run q times (q is
  // uniform, 1 for rows of up to 2048 blocks).
  const uint32_t q = (words + kWave - 1) / kWave;
  uint2 *mine = bitmap + lane * q;
#pragma unroll 1
  for (uint32_t j = 0; j < q; ++j) mine[j].x = 0;
  wave_lds_sync();
  if constexpr (kPairs) {
#pragma unroll
    for (int e = 0; e < E; e += 2)
      if (a[e] != kSentinel)
        atomicOr(&bitmap[a[e] >> 5].x, (a[e + 1] != kSentinel ? 3u : 1u) << (a[e] & 31));
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (a[e] != kSentinel) atomicOr(&bitmap[a[e] >> 5].x, 1u << (a[e] & 31));
  }
  wave_lds_sync();
  uint32_t count = 0;
#pragma unroll 1
  for (uint32_t j = 0; j < q; ++j) count += __builtin_popcount(mine[j].x);
  uint32_t total;
  uint32_t below = wave_exclusive_sum(count, lane, &total);
  if (total != static_cast<uint32_t>(n_valid)) return false;  // uniform
#pragma unroll 1
  for (uint32_t j = 0; j < q; ++j) {
    const uint32_t w = mine[j].x;
    mine[j].y = below;
    below += __builtin_popcount(w);
  }
  wave_lds_sync();
  // Rank = kept blocks in earlier words + set bits below the key in its word.
#pragma unroll
  for (int e = 0; e < E; e += (kPairs ? 2 : 1))
    if (a[e] != kSentinel) {
      const uint2 wp = bitmap[a[e] >> 5];
      const uint32_t rank = wp.y + __builtin_popcount(wp.x & ((1u << (a[e] & 31)) - 1u));
      sorted[rank] = a[e];
      if constexpr (kPairs)
        if (a[e + 1] != kSentinel) sorted[rank + 1] = a[e + 1];
    }
  wave_lds_sync();
  // Positions n_valid and above are never read from a[] afterwards.
#pragma unroll
  for (int e = 0; e < E; ++e) a[e] = sorted[lane * E + e];
  return true;
}

// One row's loaded inputs: its ks, ke and the lane's E candidates.
template <int E>
struct RowInput {
  int32_t ks, ke;
  int32_t cv[E];
};

// Issues one row's loads. Positions past L (only when E == 1: for E > 1,
// L = K * RATIO is exactly 64 * E, K being a power of two) read candidate
// K-1, a valid address, and are dropped later; offsets are 32-bit bytes from
// the row's base (K <= 1024).
template <int E>
__device__ __forceinline__ void load_row(RowInput<E> &in, const int32_t *cand, int64_t cand_stride,
                                         const int32_t *row_ks, int64_t ks_stride,
                                         const int32_t *row_ke, int64_t ke_stride, uint32_t row,
                                         int lane, int32_t L, uint32_t split) {
  in.ks = row_ks[row * ks_stride];
  in.ke = row_ke[row * ke_stride];
  const char *crow = reinterpret_cast<const char *>(cand + row * cand_stride);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int32_t i = lane * E + e;
    const uint32_t idx = static_cast<uint32_t>(E > 1 ? i : min(i, L - 1)) >> split;
    in.cv[e] = *reinterpret_cast<const int32_t *>(crow + idx * 4u);
  }
}

template <int E>
__device__ __forceinline__ void expand_row(const RowInput<E> &in, uint32_t row, int lane,
                                           int32_t L, uint32_t split, int32_t sbk,
                                           int32_t *sparse, int64_t sparse_stride, int32_t *end,
                                           int64_t end_stride, uint2 *bitmap, int32_t *sorted) {
  // ks, ke >= 0 (a precondition), so kv_len < 2^31 and max_block <= 2^28;
  // SBK is 8 or 16, a power of two.
  const int32_t ks = in.ks, ke = in.ke;
  const uint32_t sbk_shift = sbk == 16 ? 4u : 3u;
  const uint32_t kv_len = ke > ks ? static_cast<uint32_t>(ke - ks) : 0u;
  const uint32_t max_block = (kv_len + static_cast<uint32_t>(sbk) - 1u) >> sbk_shift;
  const int32_t base = ks >> sbk_shift;

  // Block of position i: (c << split) | (i & split). A candidate c >= 0 is
  // kept when that block is below max_block; c itself is checked first so
  // the shift cannot wrap (c < max_block <= 2^28), and negative c fail it as
  // unsigned values.
  int32_t a[E];
  int32_t n_valid = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int32_t i = lane * E + e;
    const uint32_t cu = static_cast<uint32_t>(in.cv[e]);
    const uint32_t block = (cu << split) | (static_cast<uint32_t>(i) & split);
    const bool keep = (E > 1 || i < L) && cu < max_block && block < max_block;
    a[e] = keep ? static_cast<int32_t>(block) : kSentinel;
    n_valid += __builtin_popcountll(__builtin_amdgcn_ballot_w64(keep));  // uniform
  }

  bool done = false;
  if (max_block <= kRankMaxBlocks) {  // uniform
    const uint32_t words = (max_block + 31u) / 32u;
    if constexpr (E >= 2) {
      done = split != 0u ? rank_sort<E, true>(a, lane, words, n_valid, bitmap, sorted)
                         : rank_sort<E, false>(a, lane, words, n_valid, bitmap, sorted);
    } else {
      done = rank_sort<E, false>(a, lane, words, n_valid, bitmap, sorted);
    }
  }
  if (!done) {
    // Bitonic sort of the 64 * E keys, ascending.
    const int32_t addr_xor32 = (lane ^ 32) << 2;
    bitonic_sort<E, 2>(a, lane, addr_xor32);
  }

  // The last kept block is the key at sorted position n_valid - 1.
  int32_t last = -1;
  if (n_valid > 0) {
    const int32_t pos = n_valid - 1;
    int32_t v = a[0];
#pragma unroll
    for (int e = 1; e < E; ++e) v = (pos % E) == e ? a[e] : v;
    last = __builtin_amdgcn_readlane(v, pos / E);
  }
  const int32_t pad = n_valid > 0 ? last + base : base;
  char *out = reinterpret_cast<char *>(sparse + row * sparse_stride);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int32_t i = lane * E + e;
    if (E > 1 || i < L)
      *reinterpret_cast<int32_t *>(out + static_cast<uint32_t>(i) * 4u) =
          i < n_valid ? a[e] + base : pad;
  }
  if (lane == 0) {
    // The last kept block starts at ks + last * SBK < ke (last < max_block),
    // so the tokens it covers are min(kv_len - last * SBK, SBK) >= 1, in
    // 32-bit arithmetic: last * SBK < kv_len < 2^31.
    const uint32_t rest = kv_len - static_cast<uint32_t>(last) * static_cast<uint32_t>(sbk);
    const int32_t fill = static_cast<int32_t>(min(rest, static_cast<uint32_t>(sbk)));
    end[row * end_stride] = n_valid > 0 ? (n_valid - 1) * sbk + fill : 0;
  }
}


// W waves per block, one row each; each wave has its own LDS share.
// Blocks are numbered XCD by XCD (xcd_block), so the rows whose ks, ke and
// end share a cache line run on one XCD and that line is fetched into one L2
// instead of eight.
template <int E, int W>
__global__ __launch_bounds__(W * kWave) void expand_kernel(
    const int32_t *cand, int64_t cand_stride, const int32_t *row_ks, int64_t ks_stride,
    const int32_t *row_ke, int64_t ke_stride, uint32_t rows, int32_t num_candidates,
    int32_t ratio, int32_t sbk, int32_t *sparse, int64_t sparse_stride, int32_t *end,
    int64_t end_stride, uint32_t xcd_shift) {
  __shared__ uint2 bitmap[W][kRankWords];
  __shared__ __align__(16) int32_t sorted[W][kWave * E];
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const uint32_t row = xcd_block(xcd_shift) * W + wave;
  if (row >= rows) return;
  const int32_t L = num_candidates * ratio;
  const uint32_t split = static_cast<uint32_t>(ratio) - 1u;  // 1 when each candidate is 2 blocks
  RowInput<E> in;
  load_row<E>(in, cand, cand_stride, row_ks, ks_stride, row_ke, ke_stride, row, lane, L, split);
  expand_row<E>(in, row, lane, L, split, sbk, sparse, sparse_stride, end, end_stride,
                bitmap[wave], sorted[wave]);
}

// Waves (rows) per block. Measured on MI355X at 16384 rows of 256 blocks:
// 1, 2 and 4 waves per block took 8.58, 8.43 and 8.45 us; two rows per wave,
// one after the other, took 11.2 us against 9.9 us for one (the rows' work
// serialises in the wave).
constexpr int kExpandWaves = 2;

template <int E>
hipError_t launch_expand_e(const ExpandArgs &x, hipStream_t stream) {
  const int32_t *cand = x.cand, *ks = x.ks, *ke = x.ke;
  int64_t cs = x.cand_stride, kss = x.ks_stride, kes = x.ke_stride, ss = x.sparse_stride,
          es = x.end_stride;
  uint32_t rows = static_cast<uint32_t>(x.rows);
  int32_t k = x.num_candidates, ratio = x.ratio, sbk = x.sparse_block;
  int32_t *sparse = x.sparse, *end = x.end;
  uint32_t xcd_shift = 0;
  const dim3 grid = xcd_grid<kExpandWaves>(rows, &xcd_shift);
  void *params[] = {&cand, &cs,    &ks,  &kss,    &ke, &kes,    &rows,
                    &k,    &ratio, &sbk, &sparse, &ss, &end,    &es, &xcd_shift};
  return hipLaunchKernel(reinterpret_cast<const void *>(expand_kernel<E, kExpandWaves>), grid,
                         dim3(kExpandWaves * kWave), params, 0, stream);
}

}  // namespace

// One wave per row; more rows than one launch takes run as several launches
// over consecutive row slices.
hipError_t launch_expand(const ExpandArgs &x, hipStream_t stream) {
  const int64_t L = static_cast<int64_t>(x.num_candidates) * x.ratio;
  return sliced(x.rows, kMaxLaunchWaves, [&](int64_t s, int64_t m) {
    ExpandArgs y = x;
    y.rows = m;
    y.cand = x.cand + s * x.cand_stride;
    y.ks = x.ks + s * x.ks_stride;
    y.ke = x.ke + s * x.ke_stride;
    y.sparse = x.sparse + s * x.sparse_stride;
    y.end = x.end + s * x.end_stride;
    return L <= 64     ? launch_expand_e<1>(y, stream)
           : L <= 128  ? launch_expand_e<2>(y, stream)
           : L <= 256  ? launch_expand_e<4>(y, stream)
           : L <= 512  ? launch_expand_e<8>(y, stream)
           : L <= 1024 ? launch_expand_e<16>(y, stream)
                       : hipErrorInvalidValue;
  });
}

}  // namespace kvrec
