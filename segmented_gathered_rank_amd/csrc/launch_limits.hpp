// Host-side limits of one kernel launch (no device code; also built by the
// host unit tests).
#pragma once

#include <cstdint>

namespace lora {

// Whether a 1-D launch of `blocks` workgroups of `threads` work-items fits a
// HIP grid, which holds at most 2^32 - 1 work-items.
inline bool grid_fits(int64_t blocks, int threads) {
  if (blocks < 1 || threads < 1) return false;
  return blocks <= static_cast<int64_t>(UINT32_MAX) / threads;
}

}  // namespace lora
