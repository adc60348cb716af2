// attn_fwd_launch.hpp -- launch entry points shared between the translation
// units of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_fwd_common.hpp"

namespace attnfwd {

// The ping-pong kernel (tile configuration 4, attn_fwd_pp.hpp) for head dim d
// (64 or 128), dtype dt (0 = fp16, 1 = bf16) and mask mode.
hipError_t launch_pingpong(int64_t d, int dt, int mask, const Params &p, int64_t grid, hipStream_t stream);

// Lockstep-kernel configurations (ids 0, 1, 2, 3, 5, 6, 7) in their own
// translation units: contiguous K/V at head dim 64 and 128, and paged K/V at
// head dim 64 and 128.
hipError_t launch_lockstep_d64(int dt, int mask, int cfg, const Params &p, int64_t grid, hipStream_t stream);
hipError_t launch_lockstep_d128(int dt, int mask, int cfg, const Params &p, int64_t grid, hipStream_t stream);
hipError_t launch_lockstep_paged64(int dt, int mask, int cfg, const Params &p, int64_t grid, hipStream_t stream);
hipError_t launch_lockstep_paged128(int dt, int mask, int cfg, const Params &p, int64_t grid, hipStream_t stream);

}  // namespace attnfwd
