// attn_fwd_launch.hpp -- launch entry points shared between the translation
// units of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_fwd_common.hpp"

namespace attnfwd {

// Lockstep-kernel configurations (ids 0 .. 4), dtype dt (0 = fp16, 1 = bf16)
// and mask mode, in their own translation units: contiguous K/V at head dim
// 64 and 128, and paged K/V at head dim 64 and 128.
hipError_t launch_lockstep_d64(int dt, int mask, int cfg, const Params &p, int64_t grid, hipStream_t stream);
hipError_t launch_lockstep_d128(int dt, int mask, int cfg, const Params &p, int64_t grid, hipStream_t stream);
hipError_t launch_lockstep_paged64(int dt, int mask, int cfg, const Params &p, int64_t grid, hipStream_t stream);
hipError_t launch_lockstep_paged128(int dt, int mask, int cfg, const Params &p, int64_t grid, hipStream_t stream);

}  // namespace attnfwd
