// worker_bf16_buf.hip -- instantiates the product kernel (worker_impl.h) for
// bf16 values and B, with B read through a buffer resource (B below 4 GiB).
#include "worker_impl.h"

namespace sdl {

hipError_t launch_bf16_buf(const WorkerConfig &cfg, const WorkerArgs &a,
                         hipStream_t s, hipEvent_t e0, hipEvent_t e1)
{
    constexpr bool BUF = true;
    switch (cfg.vec) {
    case 8: return launch_vec<SPMM_DTYPE_BF16, 8, BUF>(cfg.group, cfg.nv, a, s, e0, e1);
    case 4: return launch_vec<SPMM_DTYPE_BF16, 4, BUF>(cfg.group, cfg.nv, a, s, e0, e1);
    case 2: return launch_vec<SPMM_DTYPE_BF16, 2, BUF>(cfg.group, cfg.nv, a, s, e0, e1);
    case 1: return launch_vec<SPMM_DTYPE_BF16, 1, BUF>(cfg.group, cfg.nv, a, s, e0, e1);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_bf16_pair(const WorkerConfig &cfg, const WorkerArgs &a,
                           hipStream_t s, hipEvent_t e0, hipEvent_t e1)
{
    return launch_pair<SPMM_DTYPE_BF16, 8, true>(cfg.group, a, s, e0, e1);
}

}  // namespace sdl
