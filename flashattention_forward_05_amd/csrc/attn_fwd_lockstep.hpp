// attn_fwd_lockstep.hpp -- launch templates of the lockstep kernel
// (attn_fwd_kernel.hpp) for the tile configurations that use it.  Included by
// the translation units that each instantiate one slice of them (by head dim,
// and contiguous or paged K/V), so that the slices compile in parallel.
#pragma once

#include <hip/hip_runtime.h>

#include "attn_fwd_kernel.hpp"

namespace attnfwd {

template <int D, int DT, int MASK, int QB, int NWQ, int KSPLIT, int BN, int NSTAGE, bool PAGED>
hipError_t launch_lockstep_one(const Params &p, int64_t grid, hipStream_t stream) {
    Params args = p;
    void *argv[] = {&args};
    return hipLaunchKernel((const void *)&attn_fwd_kernel<D, DT, MASK, QB, NWQ, KSPLIT, BN, NSTAGE, PAGED>,
                           dim3((unsigned)grid), dim3(NWQ * KSPLIT * 64), argv, 0, stream);
}

// Configuration ids 0 .. 4 (the table in attn_fwd.hip); any other id is
// hipErrorInvalidValue.
template <int D, int DT, int MASK, bool PAGED>
hipError_t launch_lockstep_cfg(int cfg, const Params &p, int64_t grid, hipStream_t stream) {
    constexpr bool small = D == 64;
    switch (cfg) {
    case 0: return launch_lockstep_one<D, DT, MASK, 1, 4, 2, 64, small ? 3 : 2, PAGED>(p, grid, stream);
    case 1: return launch_lockstep_one<D, DT, MASK, 1, 8, 1, 64, 4, PAGED>(p, grid, stream);
    case 2: return launch_lockstep_one<D, DT, MASK, 1, 2, 2, small ? 64 : 32, 2, PAGED>(p, grid, stream);
    case 3: return launch_lockstep_one<D, DT, MASK, 1, 1, 1, small ? 64 : 32, 3, PAGED>(p, grid, stream);
    case 4: return launch_lockstep_one<D, DT, MASK, 1, 1, 4, small ? 64 : 32, 2, PAGED>(p, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

template <int D, bool PAGED>
hipError_t launch_lockstep_d(int dt, int mask, int cfg, const Params &p, int64_t grid, hipStream_t stream) {
    if (dt == 0) {
        switch (mask) {
        case MASK_NONE: return launch_lockstep_cfg<D, 0, MASK_NONE, PAGED>(cfg, p, grid, stream);
        case MASK_CAUSAL: return launch_lockstep_cfg<D, 0, MASK_CAUSAL, PAGED>(cfg, p, grid, stream);
        default: return launch_lockstep_cfg<D, 0, MASK_WINDOW, PAGED>(cfg, p, grid, stream);
        }
    }
    switch (mask) {
    case MASK_NONE: return launch_lockstep_cfg<D, 1, MASK_NONE, PAGED>(cfg, p, grid, stream);
    case MASK_CAUSAL: return launch_lockstep_cfg<D, 1, MASK_CAUSAL, PAGED>(cfg, p, grid, stream);
    default: return launch_lockstep_cfg<D, 1, MASK_WINDOW, PAGED>(cfg, p, grid, stream);
    }
}

}  // namespace attnfwd
