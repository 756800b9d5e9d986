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
};

namespace rf {

// Records a thread-local message and returns `s`.
rf_status fail(rf_status s, const char* fmt, ...);

// Maps the last launch error, if any, to RF_ERR_HIP.
rf_status check_launch(const char* what);

inline bool aligned16(const void* p) {
  return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

// Checks shared by the GPU entry points: plan, B, H, d, dtype, current
// device.  Returns RF_OK or the failing status.
rf_status check_call(const rf_plan* plan, int32_t B, int32_t H, int32_t d,
                     rf_dtype dtype, const char* fn);

inline int esize(rf_dtype t) { return t == RF_BF16 ? 2 : 4; }

}  // namespace rf
