// attn_fwd_pp.hip -- ping-pong kernel instantiations (tile configuration 4),
// both head dims, in a translation unit of their own so that the library's
// slices compile in parallel.
#include "attn_fwd_launch.hpp"
#include "attn_fwd_pp.hpp"

namespace attnfwd {

namespace {

template <int D, int DT, int MASK>
hipError_t launch_pp_one(const Params &p, int64_t grid, hipStream_t stream) {
    Params args = p;
    void *argv[] = {&args};
    return hipLaunchKernel((const void *)&attn_fwd_pp_kernel<D, DT, MASK>, dim3((unsigned)grid), dim3(512), argv, 0,
                           stream);
}

template <int D, int DT>
hipError_t launch_pp_mask(int mask, const Params &p, int64_t grid, hipStream_t stream) {
    switch (mask) {
    case MASK_NONE: return launch_pp_one<D, DT, MASK_NONE>(p, grid, stream);
    case MASK_CAUSAL: return launch_pp_one<D, DT, MASK_CAUSAL>(p, grid, stream);
    default: return launch_pp_one<D, DT, MASK_WINDOW>(p, grid, stream);
    }
}

}  // namespace

hipError_t launch_pingpong(int64_t d, int dt, int mask, const Params &p, int64_t grid, hipStream_t stream) {
    if (d == 64) return dt == 0 ? launch_pp_mask<64, 0>(mask, p, grid, stream) : launch_pp_mask<64, 1>(mask, p, grid, stream);
    return dt == 0 ? launch_pp_mask<128, 0>(mask, p, grid, stream) : launch_pp_mask<128, 1>(mask, p, grid, stream);
}

}  // namespace attnfwd
