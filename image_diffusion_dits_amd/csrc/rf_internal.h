// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rf.h"

// Device-side index tables of one layout (built on the host once).
struct rf_plan {
  rf_layout lay;
  rf_sizes sz;
  int device;
  int32_t* slot_src;    // [Lp] raster token of each slot, -1 for pad
  int32_t* tok_slot;    // [L]  slot of each raster token
  uint32_t* tile_bits;  // [n_tiles][4] valid-slot bitmask of each tile
  int32_t* tile_count;  // [n_tiles] valid slots per tile
  uint8_t* is_sink;     // [nb] 1 for sink blocks
  int32_t* tile_rank;   // [nb] position of each video tile in spatial-major order
};

namespace rf {

// Records a thread-local message and returns `s`.
rf_status fail(rf_status s, const char* fmt, ...);

// Maps the last launch error, if any, to RF_ERR_HIP.
rf_status check_launch(const char* what);

// Sets the dynamic-LDS limits of the mask-prediction kernels on the current
// device (called once by rf_plan_create).
rf_status prepare_mask_kernels();

inline bool aligned16(const void* p) {
  return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

// Checks shared by the GPU entry points: plan, B, H, d, dtype, current
// device.  Returns RF_OK or the failing status.
rf_status check_call(const rf_plan* plan, int32_t B, int32_t H, int32_t d,
                     rf_dtype dtype, const char* fn);

inline int esize(rf_dtype t) { return t == RF_BF16 ? 2 : 4; }

// Row of query tile `tile` in one head's kept-tile list: offset from the
// head's base and length.  row_len_video > 0: the layout rf_predict_mask
// writes (video rows of row_len_video entries, then text rows of n_tiles).
// row_len_video < 0: every row holds -row_len_video entries, the kept ids
// first (ascending) and -1 padding after them, so the length is the position
// of the first negative entry, found by binary search.
struct RowRef {
  int64_t offset;
  int32_t len;
};

__device__ inline RowRef row_ref(const int32_t* kept_head, int32_t tile, int32_t nb,
                                 int32_t row_len_video, int32_t n_tiles) {
  if (row_len_video >= 0) {
    if (tile < nb) return {int64_t(tile) * row_len_video, row_len_video};
    return {int64_t(nb) * row_len_video + int64_t(tile - nb) * n_tiles, n_tiles};
  }
  const int32_t w = -row_len_video;
  const int32_t* r = kept_head + int64_t(tile) * w;
  int32_t lo = 0, hi = w;
  while (lo < hi) {
    const int32_t mid = (lo + hi) >> 1;
    if (r[mid] >= 0) lo = mid + 1;
    else hi = mid;
  }
  return {int64_t(tile) * w, lo};
}

}  // namespace rf
