// Digit choice of one radix-select pass, shared by the PDDP split and the
// top-K selection.
#pragma once

#include "mcs_common.hpp"

namespace mcs {

// Called by all 64 lanes of one wave. hist[256] (LDS) holds the counts of
// the candidates per 8-bit digit. Visiting digits in ascending order
// (DESC = false) or descending order (DESC = true), it finds the first digit
// at which the running count reaches `remaining` (1 <= remaining <= total),
// and the lane holding it writes that digit (plus digit_base) and the count
// of the candidates visited before it (plus before_base). Same answer as a
// sequential scan.
template <bool DESC>
__device__ __forceinline__ void radix_pick(const uint32_t *hist, uint32_t remaining, uint32_t *digit_out,
                                           uint32_t *before_out, uint32_t digit_base = 0,
                                           uint32_t before_base = 0) {
  const int lane = threadIdx.x & 63;
  uint32_t c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * lane + i;  // position in visiting order
    c[i] = hist[DESC ? 255 - r : r];
  }
  const uint32_t s = c[0] + c[1] + c[2] + c[3];
  uint32_t x = s;  // inclusive scan of the lanes' sums
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  uint32_t cum = x - s;
  int found = -1;
  uint32_t before = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (found < 0 && cum + c[i] >= remaining) {
      found = i;
      before = cum;
    }
    cum += c[i];
  }
  const uint64_t b = __ballot(found >= 0);
  if (b != 0 && lane == __ffsll((unsigned long long)b) - 1) {
    const int r = 4 * lane + found;
    *digit_out = digit_base + (uint32_t)(DESC ? 255 - r : r);
    *before_out = before_base + before;
  }
}

}  // namespace mcs
