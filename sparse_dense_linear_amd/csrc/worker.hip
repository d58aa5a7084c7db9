// worker.hip -- host side of the product kernel: the choice of variant
// (lane-group width, vector width) for a call and the dispatch to the file
// that instantiates it (worker_f32.hip, worker_bf16.hip, worker_fused.hip;
// the kernels themselves are in worker_impl.h).
#include <hip/hip_runtime.h>

#include "internal.h"
#include "spmm.h"

namespace sdl {

WorkerConfig choose_worker(int dtype, int64_t N, const void *B, const float *C)
{
    const int esz = dtype == SPMM_DTYPE_BF16 ? 2 : 4;
    const uintptr_t bp = (uintptr_t)B, cp = (uintptr_t)C;
    // Widest lane vector (at most 16 bytes of B) that divides N and whose
    // B loads and C stores are aligned.
    int vec = 16 / esz;
    for (; vec > 1; vec /= 2) {
        const int64_t bbytes = (int64_t)vec * esz;
        const int64_t cbytes = (int64_t)vec * 4 < 16 ? (int64_t)vec * 4 : 16;
        if (N % vec == 0 && bp % bbytes == 0 && cp % cbytes == 0)
            break;
    }
    const int64_t vecs = (N + vec - 1) / vec;  // lane vectors per B row
    // The narrowest power-of-two group that covers a row with one vector per
    // lane: small N (one or two vectors per row) gets groups of 1 or 2 lanes
    // and 64 or 32 rows per wavefront, instead of lanes that would only
    // repeat a neighbour's load.
    int group = 1;
    while (group < 64 && group < vecs)
        group *= 2;
    int64_t nv = (vecs + group - 1) / group;
    nv = nv <= 1 ? 1 : (nv <= 2 ? 2 : 4);
    WorkerConfig cfg;
    cfg.dtype = dtype;
    cfg.vec = vec;
    cfg.group = group;
    cfg.nv = (int)nv;
    return cfg;
}

bool fused_fits(const WorkerConfig &cfg, int64_t N)
{
    // At most 1024 columns: wider bf16 rows (4 vectors per lane) spill.
    return cfg.vec == (cfg.dtype == SPMM_DTYPE_F32 ? 4 : 8) && N <= 1024 &&
           N <= (int64_t)cfg.group * cfg.vec * cfg.nv;
}

// B of at least this size (more than the Infinity Cache) takes the PAIR form.
constexpr uint64_t kPairMinBBytes = (uint64_t)256 << 20;

hipError_t launch_call(const WorkerConfig &cfg, const WorkerArgs &a,
                       hipStream_t s, hipEvent_t e0, hipEvent_t e1)
{
    // B is addressed through a buffer resource (32-bit byte offsets) when it
    // is below 4 GiB, otherwise through flat 64-bit addresses.
    const int esz = cfg.dtype == SPMM_DTYPE_BF16 ? 2 : 4;
    const uint64_t b_bytes = (uint64_t)a.K * (uint64_t)a.N * (uint64_t)esz;
    const bool buf = b_bytes <= kBufMaxBytes;
    if (a.dot_rows != nullptr) {
        // FusedMM: 16-byte vectors, the whole row in one column pass.
        if (!fused_fits(cfg, a.N) || a.dot_cols == nullptr)
            return hipErrorInvalidValue;
        return buf ? launch_fused_buf(cfg, a, s, e0, e1) : launch_fused_flat(cfg, a, s, e0, e1);
    }
    // B larger than the Infinity Cache, read through a buffer resource, with
    // rows of 512 bytes (two column passes of 16 lanes): the PAIR form
    // (medium rows four at a time, one column half per item).  Rows of 1 KB
    // keep the one-pass form: the skewed bf16 workload (N = 512), whose
    // hub chunks and short tiles would then take two column passes each,
    // was 5 % slower in the PAIR form.
    const int64_t half_vecs = cfg.vec > 0 ? a.N / 2 / cfg.vec : 0;
    if (buf && b_bytes >= kPairMinBBytes && cfg.vec * esz == 16 && a.N % (2 * cfg.vec) == 0 &&
        half_vecs == 16) {
        WorkerConfig pc = cfg;
        pc.group = (int)half_vecs;
        pc.nv = 1;
        return cfg.dtype == SPMM_DTYPE_F32 ? launch_f32_pair(pc, a, s, e0, e1)
                                           : launch_bf16_pair(pc, a, s, e0, e1);
    }
    if (cfg.dtype == SPMM_DTYPE_F32)
        return buf ? launch_f32_buf(cfg, a, s, e0, e1) : launch_f32_flat(cfg, a, s, e0, e1);
    return buf ? launch_bf16_buf(cfg, a, s, e0, e1) : launch_bf16_flat(cfg, a, s, e0, e1);
}

}  // namespace sdl
