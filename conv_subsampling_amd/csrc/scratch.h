// The library-owned device scratch of the allocation-free entry point
// (scratch.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace dw {

// Size of the per-device scratch array: 16 MiB.  The conv2d backward's
// fp64 partials take (P + chunks) * 10 * C * 8 bytes with at most P = 256
// workgroup partials and 4 chunk rows, whatever the batch size, so this
// holds them for C up to 806 channels.
constexpr size_t kScratchBytes = (size_t)16 << 20;

// The device address of the current device's scratch array, looked up with
// hipGetSymbolAddress on this device's first call and kept.  Thread-safe.
hipError_t scratch_on_current_device(void** out);

}  // namespace dw
