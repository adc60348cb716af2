// attn_fwd_pipe.hip -- launches of the in-wave pipelined attention kernels
// (attn_fwd_pipe.hpp).  Built as its own translation unit with MFMA results
// kept in ordinary VGPRs (-mllvm -amdgpu-mfma-vgpr-form=1): the softmax reads
// the S^T accumulators with plain vector instructions instead of copying them
// out of accumulation registers every tile.
#include <hip/hip_runtime.h>

#include "attn_fwd_launch.hpp"
#include "attn_fwd_pipe.hpp"

namespace attnfwd {
namespace {

template <int D, int DT, int MASK, int QB, int NWQ, int KSPLIT, int BN>
hipError_t launch_pipe(const Params &p, int64_t grid, hipStream_t stream) {
    Params args = p;
    void *argv[] = {&args};
    return hipLaunchKernel((const void *)&attn_fwd_pipe_kernel<D, DT, MASK, QB, NWQ, KSPLIT, BN>,
                           dim3((unsigned)grid), dim3(NWQ * KSPLIT * 64), argv, 0, stream);
}

template <int D, int DT, int MASK>
hipError_t pipe_cfg(int cfg, const Params &p, int64_t grid, hipStream_t stream) {
    constexpr bool small = D == 64;
    switch (cfg) {
    case 6: return launch_pipe<D, DT, MASK, 1, 4, 1, small ? 64 : 32>(p, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

template <int D, int DT>
hipError_t pipe_mask(int mask, int cfg, const Params &p, int64_t grid, hipStream_t stream) {
    switch (mask) {
    case MASK_NONE: return pipe_cfg<D, DT, MASK_NONE>(cfg, p, grid, stream);
    case MASK_CAUSAL: return pipe_cfg<D, DT, MASK_CAUSAL>(cfg, p, grid, stream);
    default: return pipe_cfg<D, DT, MASK_WINDOW>(cfg, p, grid, stream);
    }
}

}  // namespace

hipError_t launch_pipelined(int64_t d, int dt, int mask, int cfg, const Params &p, int64_t grid,
                            hipStream_t stream) {
    if (d == 64) return dt == 0 ? pipe_mask<64, 0>(mask, cfg, p, grid, stream) : pipe_mask<64, 1>(mask, cfg, p, grid, stream);
    return dt == 0 ? pipe_mask<128, 0>(mask, cfg, p, grid, stream) : pipe_mask<128, 1>(mask, cfg, p, grid, stream);
}

}  // namespace attnfwd
