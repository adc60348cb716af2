// attn_fwd_paged64.hip -- lockstep kernel instantiations for paged K/V, head dim 64
// (a translation unit of its own so that the library's slices compile in
// parallel).
#include "attn_fwd_launch.hpp"
#include "attn_fwd_lockstep.hpp"

namespace attnfwd {

hipError_t launch_lockstep_paged64(int dt, int mask, int cfg, const Params &p, int64_t grid, hipStream_t stream) {
    return launch_lockstep_d<64, true>(dt, mask, cfg, p, grid, stream);
}

}  // namespace attnfwd
