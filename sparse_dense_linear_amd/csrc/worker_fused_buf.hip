// worker_fused_buf.hip -- instantiates the product kernel (worker_impl.h) for
// the FusedMM form (16-byte vectors of fp32 or bf16), with B read through a buffer resource (B below 4 GiB).
#include "worker_impl.h"

namespace sdl {

hipError_t launch_fused_buf(const WorkerConfig &cfg, const WorkerArgs &a,
                         hipStream_t s, hipEvent_t e0, hipEvent_t e1)
{
    constexpr bool BUF = true;
    if (cfg.dtype == SPMM_DTYPE_F32)
        return launch_vec<SPMM_DTYPE_F32, 4, BUF, true>(cfg.group, cfg.nv, a, s, e0, e1);
    return launch_vec<SPMM_DTYPE_BF16, 8, BUF, true>(cfg.group, cfg.nv, a, s, e0, e1);
}

}  // namespace sdl
