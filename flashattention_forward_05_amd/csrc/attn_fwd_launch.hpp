// attn_fwd_launch.hpp -- launch entry points shared between the translation
// units of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_fwd_common.hpp"

namespace attnfwd {

// Launch tile configuration cfg (6) of the in-wave pipelined kernel for
// head dim d (64 or 128), dtype dt (0 = fp16, 1 = bf16) and mask mode.
hipError_t launch_pipelined(int64_t d, int dt, int mask, int cfg, const Params &p, int64_t grid,
                            hipStream_t stream);

}  // namespace attnfwd
