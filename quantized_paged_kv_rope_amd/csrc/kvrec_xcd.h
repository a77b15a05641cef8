// kvrec_xcd.h - XCD-aware block numbering shared by the kernels (internal;
// not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvrec {

// Workgroups are handed to the 8 XCDs round-robin (block b runs on XCD
// b % 8), and each XCD has its own L2. Blocks are renumbered so that each XCD
// runs chunks of C = 2^xcd_shift consecutive (logical) blocks: the i-th block
// on XCD x is block ((i / C) * 8 + x) * C + i % C. A chunk keeps the small
// per-token arrays (slots, positions, indices: 16..32 tokens per 128 B line)
// and the 8 B / 16 B scale rows of neighbouring tokens in one L2 instead of
// eight. C is 512 blocks (chunks of 512 measured 1-2% faster than one
// contiguous range per XCD for single launches on clean caches: insert 89.7
// -> 87.5 us, gather 68.4 -> 66.9 us at 262144 tokens; the same back to back;
// chunks of 4096 made the gather slower, 72 us, and the insert + gather step
// took 139.5 us with chunks of 512 against 140-142 with 256 or 1024), or for
// grids of up to
// 8 * 512 blocks the power of two that gives each XCD one chunk. The grid is
// padded to whole chunks on every XCD; the padding blocks find no work.
constexpr int kXcds = 8;
constexpr uint32_t kXcdChunkShift = 9;  // 512 blocks

__device__ __forceinline__ uint32_t xcd_block(uint32_t xcd_shift) {
  const uint32_t b = blockIdx.x;
  const uint32_t x = b % kXcds, i = b / kXcds;
  return (((i >> xcd_shift) * kXcds + x) << xcd_shift) + (i & ((1u << xcd_shift) - 1u));
}

// Grid of `waves` (>= 1) waves in blocks of W, padded to whole chunks on
// every XCD, and the chunk's log2 (see xcd_block).
template <int W>
inline dim3 xcd_grid(int64_t waves, uint32_t *xcd_shift) {
  const int64_t blocks = (waves + W - 1) / W;
  const int64_t per_xcd = (blocks + kXcds - 1) / kXcds;
  uint32_t shift = 0;
  while (shift < kXcdChunkShift && (int64_t{1} << shift) < per_xcd) ++shift;
  const int64_t chunk = int64_t{1} << shift;
  const int64_t chunks = (blocks + kXcds * chunk - 1) / (kXcds * chunk);
  *xcd_shift = shift;
  return dim3(static_cast<uint32_t>(chunks * chunk * kXcds));
}

// Runs launch(first_row, rows) over consecutive slices of at most `slice`
// rows, stopping at the first launch error.
template <typename F>
hipError_t sliced(int64_t n, int64_t slice, F launch) {
  for (int64_t s = 0; s < n; s += slice) {
    const hipError_t err = launch(s, n - s < slice ? n - s : slice);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace kvrec
