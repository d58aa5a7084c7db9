// worker_f32_buf.hip -- instantiates the product kernel (worker_impl.h) for
// fp32 values and B, with B read through a buffer resource (B below 4 GiB).
#include "worker_impl.h"

namespace sdl {

hipError_t launch_f32_buf(const WorkerConfig &cfg, const WorkerArgs &a,
                         hipStream_t s, hipEvent_t e0, hipEvent_t e1)
{
    constexpr bool BUF = true;
    switch (cfg.vec) {
    case 4: return launch_vec<SPMM_DTYPE_F32, 4, BUF>(cfg.group, cfg.nv, a, s, e0, e1);
    case 2: return launch_vec<SPMM_DTYPE_F32, 2, BUF>(cfg.group, cfg.nv, a, s, e0, e1);
    case 1: return launch_vec<SPMM_DTYPE_F32, 1, BUF>(cfg.group, cfg.nv, a, s, e0, e1);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_f32_pair(const WorkerConfig &cfg, const WorkerArgs &a,
                          hipStream_t s, hipEvent_t e0, hipEvent_t e1)
{
    return launch_pair<SPMM_DTYPE_F32, 4, true>(cfg.group, a, s, e0, e1);
}

}  // namespace sdl
