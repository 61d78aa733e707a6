// Host entry of the composed (one primitive per launch) baseline chains.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fnorm {
namespace composed {

// Workspace bytes the chain needs: fp32 intermediates of the whole tensor
// (one for RMSNorm, two for LayerNorm) plus per-row scalars, each region
// 256-byte aligned.
int64_t workspace_bytes(bool layer, int64_t rows, int64_t width);

// Queues the chain on `stream`.  vec4: width % 4 == 0 and every pointer
// 16-byte aligned (4-element packs), else scalar accesses.
hipError_t run(bool layer, const void* x, const void* w, const void* b, void* y, int64_t rows,
               int64_t width, float eps, int dtype, bool vec4, void* workspace, int cus,
               void* stream);

}  // namespace composed
}  // namespace fnorm
