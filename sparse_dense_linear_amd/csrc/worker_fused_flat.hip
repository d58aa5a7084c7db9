// worker_fused_flat.hip -- instantiates the product kernel (worker_impl.h) for
// the FusedMM form (16-byte vectors of fp32 or bf16), with B read through 64-bit addresses.
#include "worker_impl.h"

namespace sdl {

hipError_t launch_fused_flat(const WorkerConfig &cfg, const WorkerArgs &a,
                         hipStream_t s, hipEvent_t e0, hipEvent_t e1)
{
    constexpr bool BUF = false;
    if (cfg.dtype == SPMM_DTYPE_F32)
        return launch_vec<SPMM_DTYPE_F32, 4, BUF, true>(cfg.group, cfg.nv, a, s, e0, e1);
    return launch_vec<SPMM_DTYPE_BF16, 8, BUF, true>(cfg.group, cfg.nv, a, s, e0, e1);
}

}  // namespace sdl
