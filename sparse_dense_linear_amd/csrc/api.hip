// api.hip -- host side of the C ABI declared in include/spmm.h.
//
// Checks arguments before any HIP call, resolves the routing thresholds,
// takes the stream's scratch space (the row plan), enqueues the one kernel
// that plans and computes the product, and returns without waiting for the
// device.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "internal.h"
#include "spmm.h"

using namespace sdl;

namespace {

thread_local std::string g_last_error;

spmm_status_t fail(spmm_status_t st, const std::string &msg)
{
    g_last_error = msg;
    return st;
}

spmm_status_t fail_hip(hipError_t err, const char *where)
{
    g_last_error = std::string(where) + ": " + hipGetErrorString(err);
    return SPMM_ERROR_HIP;
}

constexpr int64_t kMaxIndex = (int64_t)1 << 31;  // int32 rows / columns

// ----------------------------------------------------------- thresholds

// Gathers a lane keeps in flight for a worker variant (see worker.hip).
int unroll_of(int nv) { return nv == 1 ? 8 : (nv == 2 ? 4 : 2); }

// Hub rows: used when B is larger than the 256 MB Infinity Cache
// (kHubMinBBytes); a slab holds kSlabBytes of B's rows, and a row is a hub
// row when it has at least kHubEntriesPerSlab entries per slab on average
// (so a hub chunk is worth its search and its atomic adds).  Measured: the
// skewed 1 GiB-B workload 17.8 -> 6.9 ms (hub threshold 8192-16384 and 2 MiB
// slabs best; 1 and 4 MiB slabs 7-11 % slower); on the power-law workload
// (64 MiB B, which the Infinity Cache holds) hub rows gained nothing and
// varied more from call to call, so below 256 MiB they stay off.
constexpr int64_t kHubMinBBytes = (int64_t)256 << 20;
constexpr int64_t kSlabBytes = (int64_t)2 << 20;
constexpr int64_t kHubEntriesPerSlab = 32;

// fp32 FusedMM runs in one launch for N up to kFusedShortRowsMaxN, and for
// wider rows only when rows hold at least kFusedLongRowMean entries on
// average.
constexpr int64_t kFusedShortRowsMaxN = 64;
constexpr int64_t kFusedLongRowMean = 32;

spmm_status_t resolve(int32_t dtype, int64_t K, int64_t N, const spmm_tuning_t *req,
                      spmm_tuning_t *out)
{
    if (dtype != SPMM_DTYPE_F32 && dtype != SPMM_DTYPE_BF16)
        return fail(SPMM_ERROR_INVALID_VALUE, "unknown dtype");
    if (N < 0 || N >= kMaxIndex)
        return fail(SPMM_ERROR_INVALID_VALUE, "N out of range");
    if (K < 0 || K >= kMaxIndex)
        return fail(SPMM_ERROR_INVALID_VALUE, "K out of range");
    if (req && req->reserved != 0)
        return fail(SPMM_ERROR_INVALID_VALUE, "spmm_tuning_t.reserved must be 0");
    // Nominal variant for this N (aligned pointers): R groups of G lanes.
    const WorkerConfig cfg = choose_worker(dtype, N > 0 ? N : 1, nullptr, nullptr);
    const int R = kWave / cfg.group;
    const int U = unroll_of(cfg.nv);
    // Defaults: a short row fits two unrolled gather rounds of one group; a
    // wavefront item (medium row or long-row chunk) holds 1024 / R entries
    // (kept within [128, 4096]), so each of its R groups gathers about 1024
    // / R^2 rows of B: wide rows of B (few groups) get long items, narrow
    // rows short ones, which keeps an item's chain of dependent gathers
    // short where many items run side by side.  Measured on the power-law
    // (R = 4) and the pruned and skewed (R = 1) workloads.
    int64_t chunk = 1024 / R;
    chunk = chunk < 128 ? 128 : (chunk > 4096 ? 4096 : chunk);
    spmm_tuning_t t;
    t.short_max = 2 * U;
    t.chunk_nnz = (int32_t)chunk;
    t.medium_max = (int32_t)chunk;
    const int64_t esz = dtype == SPMM_DTYPE_BF16 ? 2 : 4;
    const int64_t row_bytes = (N > 0 ? N : 1) * esz;
    int64_t slab = kSlabBytes / row_bytes;
    slab = slab < 1 ? 1 : (slab > kMaxIndex - 1 ? kMaxIndex - 1 : slab);
    t.slab_rows = (int32_t)slab;
    t.hub_min = INT32_MAX;   // no hub rows
    t.reserved = 0;
    if (req) {
        if (req->short_max >= 0)
            t.short_max = req->short_max;
        if (req->medium_max >= 0)
            t.medium_max = req->medium_max;
        if (req->chunk_nnz > 0)
            t.chunk_nnz = req->chunk_nnz;
        if (req->slab_rows > 0)
            t.slab_rows = req->slab_rows;
    }
    if ((uint64_t)K * (uint64_t)row_bytes >= (uint64_t)kHubMinBBytes) {  // < 2^64: no wrap
        const int64_t n_slabs = (K + t.slab_rows - 1) / t.slab_rows;
        int64_t h = kHubEntriesPerSlab * n_slabs;
        h = h < t.medium_max ? t.medium_max : (h > INT32_MAX ? INT32_MAX : h);
        t.hub_min = (int32_t)h;
    }
    if (req && req->hub_min >= 0)
        t.hub_min = req->hub_min;
    // A short tile stages at most kShortCap entries and holds at least R
    // rows, so a short row may hold at most kShortCap / R entries; longer
    // rows go to the medium kind.
    if (t.short_max > kShortCap / R)
        t.short_max = kShortCap / R;
    if (t.short_max > t.medium_max)
        return fail(SPMM_ERROR_INVALID_VALUE, "short_max > medium_max");
    *out = t;
    return SPMM_SUCCESS;
}

// The kernels' form of resolved thresholds for a call with K rows of B.
Thresholds thresholds_of(const spmm_tuning_t &t, int64_t K)
{
    Thresholds th;
    th.short_max = t.short_max;
    th.medium_max = t.medium_max;
    th.chunk_nnz = t.chunk_nnz;
    th.hub_top = t.hub_min > t.medium_max ? t.hub_min : t.medium_max;
    th.slab_rows = t.slab_rows;
    th.n_slabs = (int32_t)((K + t.slab_rows - 1) / t.slab_rows);
    return th;
}

// ------------------------------------------------------------- scratch

struct DevicePool {
    bool ready = false;
    hipMemPool_t pool = nullptr;
};

std::mutex g_pool_mu;
std::vector<DevicePool> g_pools;

hipError_t pool_for_device(int dev, hipMemPool_t *out)
{
    std::lock_guard<std::mutex> lock(g_pool_mu);
    if ((int)g_pools.size() <= dev)
        g_pools.resize(dev + 1);
    DevicePool &p = g_pools[dev];
    if (!p.ready) {
        hipMemPoolProps props;
        memset(&props, 0, sizeof props);
        props.allocType = hipMemAllocationTypePinned;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipError_t err = hipMemPoolCreate(&p.pool, &props);
        if (err != hipSuccess)
            return err;
        // Keep freed blocks cached in the pool instead of returning them to
        // the device at every synchronisation.
        uint64_t keep = UINT64_MAX;
        err = hipMemPoolSetAttribute(p.pool, hipMemPoolAttrReleaseThreshold, &keep);
        if (err != hipSuccess)
            return err;
        p.ready = true;
    }
    *out = p.pool;
    return hipSuccess;
}

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Byte offsets of the plan arrays inside one scratch block (see
// PlanBuffers).  The block is zeroed when created; words are tagged with a
// per-call epoch, so a block can serve calls of any M up to its size.
struct ScratchLayout {
    int64_t counts, faults, queues, agg, medium_rows, long_row,
        long_first, chunk_row, chunk_k, total;
    int64_t chunk_cap;
    int64_t rows;
};

ScratchLayout scratch_layout(int64_t M)
{
    ScratchLayout l;
    l.rows = M;
    int64_t off = 0;
    l.counts = off;
    off = align_up(off + 5 * 8, 256);
    l.faults = off;
    off = align_up(off + 4, 256);
    l.queues = off;
    off = align_up(off + 4 * 2 * kQueues * kQueueStride, 256);
    l.agg = off;
    off = align_up(off + 8 * kPlanCounts * kPlanMaxBlocks, 256);
    l.medium_rows = off;
    off = align_up(off + 8 * M, 256);
    l.long_row = off;
    off = align_up(off + 8 * M, 256);
    l.long_first = off;
    off = align_up(off + 8 * M, 256);
    l.chunk_cap = M + kChunkTableSlack;
    l.chunk_row = off;
    off = align_up(off + 8 * l.chunk_cap, 256);
    l.chunk_k = off;
    off = align_up(off + 8 * l.chunk_cap, 256);
    l.total = off;
    return l;
}

PlanBuffers carve(char *base, const ScratchLayout &l)
{
    PlanBuffers b;
    b.counts = (uint64_t *)(base + l.counts);
    b.agg = (uint64_t *)(base + l.agg);
    b.medium_rows = (uint64_t *)(base + l.medium_rows);
    b.long_row = (uint64_t *)(base + l.long_row);
    b.long_first = (uint64_t *)(base + l.long_first);
    b.chunk_row = (uint64_t *)(base + l.chunk_row);
    b.chunk_k = (uint64_t *)(base + l.chunk_k);
    b.faults = (uint32_t *)(base + l.faults);
    b.queues = (uint32_t *)(base + l.queues);
    b.chunk_cap = l.chunk_cap;
    b.rows = l.rows;
    return b;
}

bool test_fail_alloc()
{
    const char *v = getenv("SPMM_TEST_FAIL_ALLOC");
    return v != nullptr && v[0] == '1';
}

// Per-(device, stream) state: the plan scratch block, the work buffer and
// the last epoch.  A call holds the state's mutex from the moment it picks
// its epoch and buffers until all of its launches are enqueued, so calls
// made on one stream from several host threads reach the stream in epoch
// order, and a buffer replaced by a growing call is freed (stream-ordered)
// only after every launch that uses it has been enqueued.  Calls on
// different streams never share scratch.  Each call on a block gets the next
// epoch; epoch 0 never occurs, so a zeroed block holds no valid word.
// States are never deleted (spmm_stream_release empties one), so a pointer
// to one stays valid for the life of the process.
struct StreamState {
    int dev = 0;
    hipStream_t stream = nullptr;
    std::mutex mu;
    void *scratch = nullptr;    // plan scratch block (zeroed when created)
    size_t scratch_size = 0;
    uint32_t epoch = 0;         // last epoch used on the block
    uint32_t faults_seen = 0;   // the block's fault count at the last query
    void *aux = nullptr;        // work buffer (FusedMM values, carry slots)
    size_t aux_size = 0;
};

std::mutex g_registry_mu;
std::vector<std::unique_ptr<StreamState>> g_streams;

StreamState *stream_state(int dev, hipStream_t stream, bool create)
{
    std::lock_guard<std::mutex> lock(g_registry_mu);
    for (auto &e : g_streams)
        if (e->dev == dev && e->stream == stream)
            return e.get();
    if (!create)
        return nullptr;
    g_streams.emplace_back(new StreamState);
    g_streams.back()->dev = dev;
    g_streams.back()->stream = stream;
    return g_streams.back().get();
}

hipError_t fresh_block(int dev, hipStream_t stream, size_t size, bool zero, void **out)
{
    hipMemPool_t pool;
    hipError_t err = pool_for_device(dev, &pool);
    if (err != hipSuccess)
        return err;
    void *ptr = nullptr;
    err = hipMallocFromPoolAsync(&ptr, size, pool, stream);
    if (err != hipSuccess)
        return err;
    if (ptr == nullptr)
        return hipErrorOutOfMemory;
    if (zero && (err = hipMemsetAsync(ptr, 0, size, stream)) != hipSuccess) {
        (void)hipFreeAsync(ptr, stream);  // the memset's error is the one to report
        return err;
    }
    *out = ptr;
    return hipSuccess;
}

// Scratch block of at least `need` bytes for the stream of `ss` (whose
// mutex the caller holds), and the epoch the caller's launch must use.  A
// block that is too small (or whose epochs are used up) is replaced: the
// larger one is allocated and zeroed, the old one freed, all in stream
// order after the launches already enqueued on the stream.
hipError_t scratch_for(StreamState &ss, size_t need, void **out, uint32_t *epoch)
{
    if (ss.scratch && ss.scratch_size >= need && ss.epoch != UINT32_MAX) {
        *out = ss.scratch;
        *epoch = ++ss.epoch;
        return hipSuccess;
    }
    size_t size = need;
    if (ss.scratch && size < ss.scratch_size + ss.scratch_size / 4)
        size = ss.scratch_size + ss.scratch_size / 4;
    void *ptr = nullptr;
    hipError_t err = fresh_block(ss.dev, ss.stream, size, true, &ptr);
    if (err != hipSuccess)
        return err;
    if (ss.scratch) {
        // the fault count goes on in the new block (the count only grows;
        // queries report what it gained since the last one)
        const size_t f = (size_t)scratch_layout(0).faults;
        err = hipMemcpyAsync((char *)ptr + f, (char *)ss.scratch + f, sizeof(uint32_t),
                             hipMemcpyDeviceToDevice, ss.stream);
        if (err != hipSuccess) {
            (void)hipFreeAsync(ptr, ss.stream);
            return err;
        }
        // the old block goes back after the calls that use it; a failed
        // free would only leak it, the new block is in place either way
        (void)hipFreeAsync(ss.scratch, ss.stream);
    }
    ss.scratch = ptr;
    ss.scratch_size = size;
    ss.epoch = 1;
    *out = ptr;
    *epoch = 1;
    return hipSuccess;
}

// The stream's work buffer, for arrays whose contents do not outlive a call
// (FusedMM's values, the element-balanced kernel's carry slots).  It only
// grows; the caller holds the state's mutex.  Not cleared (every call writes
// what it reads).
hipError_t aux_for(StreamState &ss, size_t need, void **out)
{
    if (ss.aux && ss.aux_size >= need) {
        *out = ss.aux;
        return hipSuccess;
    }
    size_t size = need;
    if (ss.aux && size < ss.aux_size + ss.aux_size / 4)
        size = ss.aux_size + ss.aux_size / 4;
    void *ptr = nullptr;
    hipError_t err = fresh_block(ss.dev, ss.stream, size, false, &ptr);
    if (err != hipSuccess)
        return err;
    if (ss.aux)
        (void)hipFreeAsync(ss.aux, ss.stream);  // as for the scratch block
    ss.aux = ptr;
    ss.aux_size = size;
    *out = ptr;
    return hipSuccess;
}

// ------------------------------------------------- fixed scratch (no allocation)

// spmm_csr_tuned_noalloc takes its plan scratch from this fixed array
// instead of the per-stream pool, so that it never allocates.  Every GPU the
// library runs on holds its own copy (the array is part of the library's
// device code object) until the process ends; every no-allocation call on a
// GPU shares that GPU's copy.  The array is zero when the code object is
// loaded, and plan words are tagged with a per-device epoch, so nothing is
// cleared between calls; the queue counters of the next epoch are cleared by
// each call itself (as for the per-stream blocks).
constexpr size_t kFixedScratchBytes = (size_t)12 << 20;
static __device__ __align__(256) char scratch[kFixedScratchBytes];

// Host-side state of one device's copy: its device address (from
// hipGetSymbolAddress with that device current -- the array's name is not
// a device address in host code) and the last epoch used on it.  A fixed
// table, so the no-allocation path allocates nothing on the host either.
constexpr int kMaxDevices = 64;

struct FixedScratch {
    std::mutex mu;             // held from epoch choice to enqueue
    char *ptr = nullptr;       // device address of `scratch` on this device
    uint32_t epoch = 0;
    uint32_t faults_seen = 0;  // the array's fault count at the last query
};

FixedScratch g_fixed[kMaxDevices];

// Fill kernel that zeroes the array when the per-device epochs run out (a
// kernel rather than a memset, so that the call stays capturable).
__global__ void zero_fixed_scratch(uint64_t *p, int64_t words)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

// The current device's copy of the array, its address looked up on first
// use (with that device current).  Caller holds nothing.
hipError_t fixed_scratch_for(int dev, FixedScratch **out)
{
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    FixedScratch &fs = g_fixed[dev];
    std::lock_guard<std::mutex> lock(fs.mu);
    if (fs.ptr == nullptr) {
        void *p = nullptr;
        hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess)
            return err;
        if (p == nullptr)
            return hipErrorInvalidSymbol;
        fs.ptr = (char *)p;
    }
    *out = &fs;
    return hipSuccess;
}

// Largest M whose plan scratch fits the fixed array.
int64_t fixed_scratch_max_rows()
{
    int64_t lo = 0, hi = kMaxIndex - 1;
    while (lo < hi) {
        const int64_t mid = lo + (hi - lo + 1) / 2;
        if ((size_t)scratch_layout(mid).total <= kFixedScratchBytes)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// --------------------------------------------------------------- timing

// Kernel timing: the start/stop events are attached to the kernel dispatch
// packets themselves (hipExtLaunchKernel), so timing adds no packets to the
// stream.  Events are recycled through a free list.
struct TimedCall {
    hipEvent_t work0;  // start of the call's launch
    hipEvent_t work1;  // end of the call's launch
};

std::mutex g_time_mu;
bool g_timing = false;
std::vector<TimedCall> g_timed;
std::vector<hipEvent_t> g_free_events;

hipError_t take_event(hipEvent_t *ev)
{
    if (!g_free_events.empty()) {
        *ev = g_free_events.back();
        g_free_events.pop_back();
        return hipSuccess;
    }
    return hipEventCreate(ev);
}

// ---------------------------------------------------------------- calls

spmm_status_t check_args(int32_t dtype, const int32_t *rowptr, const void *B,
                         const float *C, int64_t M, int64_t K, int64_t N)
{
    if (dtype != SPMM_DTYPE_F32 && dtype != SPMM_DTYPE_BF16)
        return fail(SPMM_ERROR_INVALID_VALUE, "unknown dtype");
    if (M < 0 || K < 0 || N < 0)
        return fail(SPMM_ERROR_INVALID_VALUE, "negative size");
    if (M >= kMaxIndex || K >= kMaxIndex || N >= kMaxIndex)
        return fail(SPMM_ERROR_INVALID_VALUE, "M, K and N must be below 2^31");
    if (M == 0 || N == 0)
        return SPMM_SUCCESS;
    if (rowptr == nullptr)
        return fail(SPMM_ERROR_INVALID_VALUE, "rowptr is null");
    if (C == nullptr)
        return fail(SPMM_ERROR_INVALID_VALUE, "C is null");
    if (K > 0 && B == nullptr)
        return fail(SPMM_ERROR_INVALID_VALUE, "B is null");
    if (((uintptr_t)C) % 4 != 0)
        return fail(SPMM_ERROR_INVALID_VALUE, "C is not 4-byte aligned");
    const uintptr_t esz = dtype == SPMM_DTYPE_BF16 ? 2 : 4;
    if (((uintptr_t)B) % esz != 0)
        return fail(SPMM_ERROR_INVALID_VALUE, "B is not aligned to its element size");
    // The kernels address a row of B with a 32-bit byte stride.
    if ((uint64_t)N * esz > 0xFFFFFFFFull)
        return fail(SPMM_ERROR_UNSUPPORTED, "a row of B must be below 4 GiB");
    return SPMM_SUCCESS;
}

// The product on `stream`; the launch carries e0/e1 when given (the
// caller then records them), else this call's timing events if enabled.
spmm_status_t run_with(int32_t dtype, const int32_t *rowptr,
                       const int32_t *colind, const void *vals, const void *B,
                       float *C, int64_t M, int64_t K, int64_t N,
                       const spmm_tuning_t *tuning, void *stream_ptr,
                       bool own_events, hipEvent_t e0, hipEvent_t e1,
                       bool vals_relative = false,
                       const void *dot_rows = nullptr,
                       const void *dot_cols = nullptr,
                       StreamState *held = nullptr, int64_t vals_count = 0)
{
    spmm_status_t st = check_args(dtype, rowptr, B, C, M, K, N);
    if (st != SPMM_SUCCESS)
        return st;
    spmm_tuning_t t;
    st = resolve(dtype, K, N, tuning, &t);
    if (st != SPMM_SUCCESS)
        return st;
    if (M == 0 || N == 0)
        return SPMM_SUCCESS;
    if (test_fail_alloc())
        return fail(SPMM_ERROR_OUT_OF_MEMORY, "allocation failure forced by SPMM_TEST_FAIL_ALLOC");

    hipStream_t stream = (hipStream_t)stream_ptr;
    hipError_t err = hipSuccess;
    // `held`: the caller (FusedMM's two-launch route) holds the stream's
    // mutex already; otherwise take it here, until the launch is enqueued.
    std::unique_lock<std::mutex> guard;
    StreamState *ss = held;
    if (ss == nullptr) {
        int dev = 0;
        if ((err = hipGetDevice(&dev)) != hipSuccess)
            return fail_hip(err, "hipGetDevice");
        ss = stream_state(dev, stream, true);
        guard = std::unique_lock<std::mutex>(ss->mu);
    }
    const ScratchLayout lay = scratch_layout(M);
    void *scratch = nullptr;
    uint32_t epoch = 0;
    err = scratch_for(*ss, (size_t)lay.total, &scratch, &epoch);
    if (err == hipErrorOutOfMemory)
        return fail(SPMM_ERROR_OUT_OF_MEMORY, "scratch allocation failed");
    if (err != hipSuccess)
        return fail_hip(err, "scratch allocation");

    TimedCall tc{};
    bool timing = false;
    if (own_events) {
        tc.work0 = e0;
        tc.work1 = e1;
    } else {
        std::lock_guard<std::mutex> lock(g_time_mu);
        timing = g_timing;
        if (timing &&
            ((err = take_event(&tc.work0)) != hipSuccess ||
             (err = take_event(&tc.work1)) != hipSuccess))
            return fail_hip(err, "hipEventCreate");
    }

    WorkerArgs wa;
    wa.rowptr = rowptr;
    wa.colind = colind;
    wa.vals = vals;
    wa.vals_relative = vals_relative ? 1 : 0;
    wa.vals_count = vals_count;
    wa.B = B;
    wa.C = C;
    wa.dot_rows = dot_rows;
    wa.dot_cols = dot_cols;
    wa.M = M;
    wa.K = K;
    wa.N = N;
    wa.th = thresholds_of(t, K);
    wa.plan = carve((char *)scratch, lay);
    wa.shape = plan_shape(M);
    wa.epoch = epoch;
    wa.wait_polls = current_wait_polls();
    const WorkerConfig cfg = choose_worker(dtype, N, B, C);
    err = launch_worker(cfg, wa, stream, tc.work0, tc.work1);
    if (err != hipSuccess)
        return fail_hip(err, "worker kernel");
    if (timing) {
        std::lock_guard<std::mutex> lock(g_time_mu);
        g_timed.push_back(tc);
    }
    return SPMM_SUCCESS;
}

spmm_status_t run(int32_t dtype, const int32_t *rowptr, const int32_t *colind,
                  const void *vals, const void *B, float *C, int64_t M,
                  int64_t K, int64_t N, const spmm_tuning_t *tuning,
                  void *stream_ptr)
{
    g_last_error.clear();
    return run_with(dtype, rowptr, colind, vals, B, C, M, K, N, tuning,
                    stream_ptr, false, nullptr, nullptr);
}

// The product with the plan in the fixed scratch array: the same checks,
// thresholds and kernel as spmm_csr_tuned; no allocation of any kind.
spmm_status_t run_noalloc(int32_t dtype, const int32_t *rowptr,
                          const int32_t *colind, const void *vals, const void *B,
                          float *C, int64_t M, int64_t K, int64_t N,
                          const spmm_tuning_t *tuning, void *stream_ptr)
{
    g_last_error.clear();
    spmm_status_t st = check_args(dtype, rowptr, B, C, M, K, N);
    if (st != SPMM_SUCCESS)
        return st;
    spmm_tuning_t t;
    st = resolve(dtype, K, N, tuning, &t);
    if (st != SPMM_SUCCESS)
        return st;
    if (M == 0 || N == 0)
        return SPMM_SUCCESS;
    const ScratchLayout lay = scratch_layout(M);
    if ((size_t)lay.total > kFixedScratchBytes)
        return fail(SPMM_ERROR_UNSUPPORTED,
                    "M = " + std::to_string(M) + " needs " + std::to_string(lay.total) +
                    " bytes of plan scratch; the fixed array of the no-allocation "
                    "entry point holds " + std::to_string(kFixedScratchBytes) +
                    " (at most " + std::to_string(fixed_scratch_max_rows()) + " rows)");
    hipStream_t stream = (hipStream_t)stream_ptr;
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess)
        return fail_hip(err, "hipGetDevice");
    FixedScratch *fs = nullptr;
    if ((err = fixed_scratch_for(dev, &fs)) != hipSuccess)
        return fail_hip(err, "hipGetSymbolAddress(scratch)");
    std::lock_guard<std::mutex> guard(fs->mu);  // until the launch is enqueued
    if (fs->epoch == UINT32_MAX) {
        // epochs used up: clear every word, then start again at 1
        const int64_t words = (int64_t)(kFixedScratchBytes / 8);
        hipLaunchKernelGGL(zero_fixed_scratch, dim3(1024), dim3(256), 0, stream,
                           (uint64_t *)fs->ptr, words);
        if ((err = hipGetLastError()) != hipSuccess)
            return fail_hip(err, "clearing the fixed scratch");
        fs->epoch = 0;
        fs->faults_seen = 0;  // the fill cleared the count too
    }
    WorkerArgs wa;
    wa.rowptr = rowptr;
    wa.colind = colind;
    wa.vals = vals;
    wa.vals_relative = 0;
    wa.vals_count = 0;
    wa.B = B;
    wa.C = C;
    wa.dot_rows = nullptr;
    wa.dot_cols = nullptr;
    wa.M = M;
    wa.K = K;
    wa.N = N;
    wa.th = thresholds_of(t, K);
    wa.plan = carve(fs->ptr, lay);
    wa.shape = plan_shape(M);
    wa.epoch = ++fs->epoch;
    wa.wait_polls = current_wait_polls();
    const WorkerConfig cfg = choose_worker(dtype, N, B, C);
    err = launch_worker(cfg, wa, stream, nullptr, nullptr);
    if (err != hipSuccess)
        return fail_hip(err, "worker kernel");
    return SPMM_SUCCESS;
}

spmm_status_t launch_sddmm_checked(int32_t dtype, const int32_t *rowptr,
                                   const int32_t *colind, const void *C,
                                   const void *B, float *A, int64_t M,
                                   int64_t K, int64_t N, int64_t nnz,
                                   void *stream_ptr);

// One SDDMM call: checks, then one launch (sddmm.hip).
spmm_status_t run_sddmm(int32_t dtype, const int32_t *rowptr,
                        const int32_t *colind, const void *C, const void *B,
                        float *A, int64_t M, int64_t K, int64_t N, int64_t nnz,
                        void *stream_ptr)
{
    g_last_error.clear();
    if (dtype != SPMM_DTYPE_F32 && dtype != SPMM_DTYPE_BF16)
        return fail(SPMM_ERROR_INVALID_VALUE, "unknown dtype");
    if (M < 0 || K < 0 || N < 0 || nnz < 0)
        return fail(SPMM_ERROR_INVALID_VALUE, "negative size");
    if (M >= kMaxIndex || K >= kMaxIndex || N >= kMaxIndex || nnz >= kMaxIndex)
        return fail(SPMM_ERROR_INVALID_VALUE, "M, K, N and nnz must be below 2^31");
    if (nnz == 0)
        return SPMM_SUCCESS;
    if (M == 0)
        return fail(SPMM_ERROR_INVALID_VALUE, "nnz > 0 with M == 0");
    if (N == 0)
        return fail(SPMM_ERROR_UNSUPPORTED, "N == 0 with stored entries");
    if (rowptr == nullptr || colind == nullptr || C == nullptr || B == nullptr ||
        A == nullptr)
        return fail(SPMM_ERROR_INVALID_VALUE, "null pointer");
    const uintptr_t esz = dtype == SPMM_DTYPE_BF16 ? 2 : 4;
    if (((uintptr_t)C) % esz != 0 || ((uintptr_t)B) % esz != 0 ||
        ((uintptr_t)A) % 4 != 0)
        return fail(SPMM_ERROR_INVALID_VALUE, "operand not aligned to its element size");
    return launch_sddmm_checked(dtype, rowptr, colind, C, B, A, M, K, N, nnz,
                                stream_ptr);
}

spmm_status_t launch_sddmm_checked(int32_t dtype, const int32_t *rowptr,
                                   const int32_t *colind, const void *C,
                                   const void *B, float *A, int64_t M,
                                   int64_t K, int64_t N, int64_t nnz,
                                   void *stream_ptr)
{
    SddmmArgs a;
    a.dtype = dtype;
    a.rowptr = rowptr;
    a.colind = colind;
    a.C = C;
    a.B = B;
    a.A = A;
    a.M = M;
    a.K = K;
    a.N = N;
    a.nnz = nnz;
    hipStream_t stream = (hipStream_t)stream_ptr;
    TimedCall tc{};
    bool timing;
    hipError_t err = hipSuccess;
    {
        std::lock_guard<std::mutex> lock(g_time_mu);
        timing = g_timing;
        if (timing &&
            ((err = take_event(&tc.work0)) != hipSuccess ||
             (err = take_event(&tc.work1)) != hipSuccess))
            return fail_hip(err, "hipEventCreate");
    }
    err = launch_sddmm(a, stream, tc.work0, tc.work1);
    if (err != hipSuccess)
        return fail_hip(err, "sddmm kernel");
    if (timing) {
        std::lock_guard<std::mutex> lock(g_time_mu);
        g_timed.push_back(tc);
    }
    return SPMM_SUCCESS;
}

// FusedMM: E_i = sum_p <C_i, B_j> D_j.  One launch of the product kernel
// in its FusedMM form when the shape allows (each value formed where it is
// used); otherwise the SDDMM values go to a stream-ordered scratch array of
// nnz floats, which the product kernel then reads as the values of A with D
// as its dense operand: two launches, the values making one round trip
// through memory.
spmm_status_t run_fusedmm(const int32_t *rowptr, const int32_t *colind,
                          const float *C, const float *B, const float *D,
                          float *E, int64_t M, int64_t K, int64_t N,
                          int64_t nnz, void *stream_ptr)
{
    g_last_error.clear();
    if (M < 0 || K < 0 || N < 0 || nnz < 0)
        return fail(SPMM_ERROR_INVALID_VALUE, "negative size");
    if (M >= kMaxIndex || K >= kMaxIndex || N >= kMaxIndex || nnz >= kMaxIndex)
        return fail(SPMM_ERROR_INVALID_VALUE, "M, K, N and nnz must be below 2^31");
    if (M == 0 || N == 0)
        return SPMM_SUCCESS;
    if (rowptr == nullptr || E == nullptr || (nnz > 0 && (colind == nullptr ||
        C == nullptr || B == nullptr || D == nullptr)))
        return fail(SPMM_ERROR_INVALID_VALUE, "null pointer");
    if ((((uintptr_t)C) | ((uintptr_t)B) | ((uintptr_t)D) | ((uintptr_t)E)) % 4 != 0)
        return fail(SPMM_ERROR_INVALID_VALUE, "operand not aligned to its element size");
    // One launch when the FusedMM form of the worker covers the shape (fp32
    // rows of at most one column pass, C and B aligned like D): each entry's
    // value is formed where it is used and never stored.  Beyond 64
    // columns that form pays only for long rows (its gathers come in pairs,
    // half as many entries in flight per lane): with a mean row of 4 entries
    // (power-law pattern) two launches were 1.5-2.2 x faster for N = 96 to
    // 1024 and one launch faster for N = 32 and 64; with 410 (pruned
    // pattern) one launch was level up to N = 512 and 1.3-1.5 x faster at
    // 768 and 1024.
    const WorkerConfig cfg = choose_worker(SPMM_DTYPE_F32, N, D, E);
    const bool long_rows = nnz >= kFusedLongRowMean * M;
    if (nnz > 0 && fused_fits(cfg, N) && (N <= kFusedShortRowsMaxN || long_rows) &&
        ((uintptr_t)C) % 16 == 0 && ((uintptr_t)B) % 16 == 0)
        return run_with(SPMM_DTYPE_F32, rowptr, colind, nullptr, D, E, M, K, N,
                        nullptr, stream_ptr, false, nullptr, nullptr, false, C, B);
    // Otherwise two launches: SDDMM into a value array, then the product,
    // both enqueued under the stream's mutex (the value array is the
    // stream's work buffer).
    hipStream_t stream = (hipStream_t)stream_ptr;
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess)
        return fail_hip(err, "hipGetDevice");
    float *vals = nullptr;
    const size_t bytes = (size_t)(nnz > 0 ? nnz : 1) * sizeof(float);
    if (test_fail_alloc())
        return fail(SPMM_ERROR_OUT_OF_MEMORY, "allocation failure forced by SPMM_TEST_FAIL_ALLOC");
    StreamState *ss = stream_state(dev, stream, true);
    std::lock_guard<std::mutex> guard(ss->mu);
    err = aux_for(*ss, bytes, (void **)&vals);
    if (err == hipErrorOutOfMemory)
        return fail(SPMM_ERROR_OUT_OF_MEMORY, "value scratch allocation failed");
    if (err != hipSuccess)
        return fail_hip(err, "value scratch allocation");

    TimedCall tc{};
    bool timing;
    {
        std::lock_guard<std::mutex> lock(g_time_mu);
        timing = g_timing;
        if (timing &&
            ((err = take_event(&tc.work0)) != hipSuccess ||
             (err = take_event(&tc.work1)) != hipSuccess))
            return fail_hip(err, "hipEventCreate");
    }
    spmm_status_t st = SPMM_SUCCESS;
    if (nnz > 0) {
        SddmmArgs a;
        a.dtype = SPMM_DTYPE_F32;
        a.rowptr = rowptr;
        a.colind = colind;
        a.C = C;
        a.B = B;
        a.A = vals;
        a.M = M;
        a.K = K;
        a.N = N;
        a.nnz = nnz;
        if ((err = launch_sddmm(a, stream, tc.work0, nullptr)) != hipSuccess)
            st = fail_hip(err, "sddmm kernel");
    }
    if (st == SPMM_SUCCESS)
        st = run_with(SPMM_DTYPE_F32, rowptr, colind, vals, D, E, M, K, N, nullptr,
                      stream_ptr, true, nnz > 0 ? nullptr : tc.work0, tc.work1,
                      true, nullptr, nullptr, ss, nnz);
    if (st == SPMM_SUCCESS && timing) {
        std::lock_guard<std::mutex> lock(g_time_mu);
        g_timed.push_back(tc);
    }
    return st;
}

// FusedMM with bf16 C, B and D (fp32 values and accumulation): the
// one-launch form when the shape allows; otherwise C, B and D are widened
// exactly into a stream-ordered fp32 copy and the fp32 FusedMM runs on it
// (the same values: every bf16 product is exact in fp32).  The copy holds
// (M + 2K) * N floats and is given back on the stream after the call.
spmm_status_t run_fusedmm_bf16(const int32_t *rowptr, const int32_t *colind,
                               const uint16_t *C, const uint16_t *B,
                               const uint16_t *D, float *E, int64_t M, int64_t K,
                               int64_t N, int64_t nnz, void *stream_ptr)
{
    g_last_error.clear();
    if (M < 0 || K < 0 || N < 0 || nnz < 0)
        return fail(SPMM_ERROR_INVALID_VALUE, "negative size");
    if (M >= kMaxIndex || K >= kMaxIndex || N >= kMaxIndex || nnz >= kMaxIndex)
        return fail(SPMM_ERROR_INVALID_VALUE, "M, K, N and nnz must be below 2^31");
    if (M == 0 || N == 0)
        return SPMM_SUCCESS;
    if (rowptr == nullptr || E == nullptr || (nnz > 0 && (colind == nullptr ||
        C == nullptr || B == nullptr || D == nullptr)))
        return fail(SPMM_ERROR_INVALID_VALUE, "null pointer");
    if ((((uintptr_t)C) | ((uintptr_t)B) | ((uintptr_t)D)) % 2 != 0 ||
        ((uintptr_t)E) % 4 != 0)
        return fail(SPMM_ERROR_INVALID_VALUE, "operand not aligned to its element size");
    if (nnz == 0)  // E = 0: the product of an empty pattern (no operand read)
        return run_with(SPMM_DTYPE_BF16, rowptr, colind, nullptr, nullptr, E, M, 0,
                        N, nullptr, stream_ptr, false, nullptr, nullptr);
    const WorkerConfig cfg = choose_worker(SPMM_DTYPE_BF16, N, D, E);
    if (fused_fits(cfg, N) && ((uintptr_t)C) % 16 == 0 && ((uintptr_t)B) % 16 == 0)
        return run_with(SPMM_DTYPE_BF16, rowptr, colind, nullptr, D, E, M, K, N,
                        nullptr, stream_ptr, false, nullptr, nullptr, false, C, B);
    // widened copy: C at 0, B and D after it, each start 256-byte aligned;
    // (M + 2K) * N * 4 can exceed 64 bits for sizes below 2^31, so it is
    // bounded before anything is sized from it
    if ((unsigned __int128)(M + 2 * K) * (unsigned __int128)N * sizeof(float) >
        ((unsigned __int128)1 << 56))
        return fail(SPMM_ERROR_OUT_OF_MEMORY, "widened operand copy above 2^56 bytes");
    hipStream_t stream = (hipStream_t)stream_ptr;
    const auto up = [](size_t b) { return (b + 255) / 256 * 256; };
    const size_t c_bytes = up((size_t)M * (size_t)N * sizeof(float));
    const size_t b_bytes = up((size_t)K * (size_t)N * sizeof(float));
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess)
        return fail_hip(err, "hipGetDevice");
    if (test_fail_alloc())
        return fail(SPMM_ERROR_OUT_OF_MEMORY, "allocation failure forced by SPMM_TEST_FAIL_ALLOC");
    char *w = nullptr;
    err = fresh_block(dev, stream, c_bytes + 2 * b_bytes, false, (void **)&w);
    if (err == hipErrorOutOfMemory)
        return fail(SPMM_ERROR_OUT_OF_MEMORY, "widened operand allocation failed");
    if (err != hipSuccess)
        return fail_hip(err, "widened operand allocation");
    float *Cw = (float *)w, *Bw = (float *)(w + c_bytes), *Dw = (float *)(w + c_bytes + b_bytes);
    spmm_status_t st = SPMM_SUCCESS;
    if ((err = launch_widen_bf16(C, Cw, M * N, stream)) != hipSuccess ||
        (err = launch_widen_bf16(B, Bw, K * N, stream)) != hipSuccess ||
        (err = launch_widen_bf16(D, Dw, K * N, stream)) != hipSuccess)
        st = fail_hip(err, "widen kernel");
    if (st == SPMM_SUCCESS)
        st = run_fusedmm(rowptr, colind, Cw, Bw, Dw, E, M, K, N, nnz, stream_ptr);
    if ((err = hipFreeAsync(w, stream)) != hipSuccess && st == SPMM_SUCCESS)
        st = fail_hip(err, "hipFreeAsync");
    return st;
}

// The element-balanced product: one launch; carry slots in the stream's
// work buffer, arrival counters in its plan scratch.
spmm_status_t run_eb(int32_t dtype, const int32_t *rowptr, const int32_t *colind,
                     const void *vals, const void *B, float *C, int64_t M,
                     int64_t K, int64_t N, void *stream_ptr)
{
    g_last_error.clear();
    spmm_status_t st = check_args(dtype, rowptr, B, C, M, K, N);
    if (st != SPMM_SUCCESS)
        return st;
    if (M == 0 || N == 0)
        return SPMM_SUCCESS;
    if (test_fail_alloc())
        return fail(SPMM_ERROR_OUT_OF_MEMORY, "allocation failure forced by SPMM_TEST_FAIL_ALLOC");
    hipStream_t stream = (hipStream_t)stream_ptr;
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess)
        return fail_hip(err, "hipGetDevice");
    const int64_t waves = eb_waves();
    if (waves <= 0)
        return fail(SPMM_ERROR_HIP, "device query failed");
    // arrival counters: the per-stream plan scratch (zeroed when created,
    // one epoch per call), enough of it for one word per span
    const ScratchLayout lay = scratch_layout(M > waves ? M : waves);
    void *scratch = nullptr;
    uint32_t epoch = 0;
    StreamState *ss = stream_state(dev, stream, true);
    std::lock_guard<std::mutex> guard(ss->mu);  // until the launch is enqueued
    err = scratch_for(*ss, (size_t)lay.total, &scratch, &epoch);
    if (err == hipErrorOutOfMemory)
        return fail(SPMM_ERROR_OUT_OF_MEMORY, "scratch allocation failed");
    if (err != hipSuccess)
        return fail_hip(err, "scratch allocation");
    const size_t bytes = (size_t)(2 * waves) * (size_t)N * sizeof(float);
    char *mem = nullptr;
    err = aux_for(*ss, bytes, (void **)&mem);
    if (err == hipErrorOutOfMemory)
        return fail(SPMM_ERROR_OUT_OF_MEMORY, "carry allocation failed");
    if (err != hipSuccess)
        return fail_hip(err, "carry allocation");
    TimedCall tc{};
    bool timing;
    {
        std::lock_guard<std::mutex> lock(g_time_mu);
        timing = g_timing;
        if (timing &&
            ((err = take_event(&tc.work0)) != hipSuccess ||
             (err = take_event(&tc.work1)) != hipSuccess))
            return fail_hip(err, "hipEventCreate");
    }
    EbArgs a;
    a.rowptr = rowptr;
    a.colind = colind;
    a.vals = vals;
    a.B = B;
    a.C = C;
    a.M = M;
    a.K = K;
    a.N = N;
    a.waves = waves;
    a.carry_val = (float *)mem;
    a.arrive = carve((char *)scratch, lay).medium_rows;
    a.queues = carve((char *)scratch, lay).queues;
    a.epoch = epoch;
    const WorkerConfig cfg = choose_worker(dtype, N, B, C);
    err = launch_eb(cfg, a, stream, tc.work0, tc.work1);
    if (err != hipSuccess)
        return fail_hip(err, "element-balanced kernel");
    if (timing) {
        std::lock_guard<std::mutex> lock(g_time_mu);
        g_timed.push_back(tc);
    }
    return SPMM_SUCCESS;
}

// Bound of the product's waits for plan entries, read by every call as it
// is enqueued (lowered only by spmm_debug_set_wait_polls).
std::atomic<int32_t> g_wait_polls{kWaitPolls};

// Reads the fault count kept in a plan scratch block, in the order of
// `stream`, and returns what it gained since the last query (*seen).  The
// device only ever adds to the count, so nothing is written back and no
// increment made during the read is lost.
hipError_t take_fault_count(char *block, hipStream_t stream, uint32_t *seen, uint32_t *out)
{
    const uint32_t *word = (const uint32_t *)(block + scratch_layout(0).faults);
    uint32_t v = 0;
    hipError_t err;
    if ((err = hipMemcpyAsync(&v, word, sizeof v, hipMemcpyDeviceToHost, stream)) != hipSuccess ||
        (err = hipStreamSynchronize(stream)) != hipSuccess)
        return err;
    *out = v - *seen;  // modulo 2^32
    *seen = v;
    return hipSuccess;
}

}  // namespace

int32_t sdl::current_wait_polls() { return g_wait_polls.load(std::memory_order_relaxed); }

extern "C" {

spmm_status_t spmm_csr_eb(int32_t dtype, const int32_t *rowptr,
                          const int32_t *colind, const void *vals,
                          const void *B, float *C, int64_t M, int64_t K,
                          int64_t N, void *stream)
{
    return run_eb(dtype, rowptr, colind, vals, B, C, M, K, N, stream);
}

spmm_status_t fusedmm_csr_f32(const int32_t *rowptr, const int32_t *colind,
                              const float *C, const float *B, const float *D,
                              float *E, int64_t M, int64_t K, int64_t N,
                              int64_t nnz, void *stream)
{
    return run_fusedmm(rowptr, colind, C, B, D, E, M, K, N, nnz, stream);
}

spmm_status_t fusedmm_csr_bf16in_f32acc(const int32_t *rowptr,
                                        const int32_t *colind, const uint16_t *C,
                                        const uint16_t *B, const uint16_t *D,
                                        float *E, int64_t M, int64_t K,
                                        int64_t N, int64_t nnz, void *stream)
{
    return run_fusedmm_bf16(rowptr, colind, C, B, D, E, M, K, N, nnz, stream);
}

spmm_status_t sddmm_csr_f32(const int32_t *rowptr, const int32_t *colind,
                            const float *C, const float *B, float *A,
                            int64_t M, int64_t K, int64_t N, int64_t nnz,
                            void *stream)
{
    return run_sddmm(SPMM_DTYPE_F32, rowptr, colind, C, B, A, M, K, N, nnz, stream);
}

spmm_status_t sddmm_csr_bf16in_f32acc(const int32_t *rowptr,
                                      const int32_t *colind, const uint16_t *C,
                                      const uint16_t *B, float *A, int64_t M,
                                      int64_t K, int64_t N, int64_t nnz,
                                      void *stream)
{
    return run_sddmm(SPMM_DTYPE_BF16, rowptr, colind, C, B, A, M, K, N, nnz, stream);
}

spmm_status_t spmm_csr_f32(const int32_t *rowptr, const int32_t *colind,
                           const float *vals, const float *B, float *C,
                           int64_t M, int64_t K, int64_t N, void *stream)
{
    return run(SPMM_DTYPE_F32, rowptr, colind, vals, B, C, M, K, N, nullptr,
               stream);
}

spmm_status_t spmm_csr_bf16in_f32acc(const int32_t *rowptr,
                                     const int32_t *colind,
                                     const uint16_t *vals, const uint16_t *B,
                                     float *C, int64_t M, int64_t K,
                                     int64_t N, void *stream)
{
    return run(SPMM_DTYPE_BF16, rowptr, colind, vals, B, C, M, K, N, nullptr,
               stream);
}

spmm_status_t spmm_csr_tuned(int32_t dtype, const int32_t *rowptr,
                             const int32_t *colind, const void *vals,
                             const void *B, float *C, int64_t M, int64_t K,
                             int64_t N, const spmm_tuning_t *tuning,
                             void *stream)
{
    return run(dtype, rowptr, colind, vals, B, C, M, K, N, tuning, stream);
}

spmm_status_t spmm_csr_tuned_noalloc(int32_t dtype, const int32_t *rowptr,
                                     const int32_t *colind, const void *vals,
                                     const void *B, float *C, int64_t M,
                                     int64_t K, int64_t N,
                                     const spmm_tuning_t *tuning, void *stream)
{
    return run_noalloc(dtype, rowptr, colind, vals, B, C, M, K, N, tuning, stream);
}

spmm_status_t spmm_resolve_tuning(int32_t dtype, int64_t K, int64_t N,
                                  const spmm_tuning_t *requested,
                                  spmm_tuning_t *resolved)
{
    g_last_error.clear();
    if (resolved == nullptr)
        return fail(SPMM_ERROR_INVALID_VALUE, "resolved is null");
    return resolve(dtype, K, N, requested, resolved);
}

spmm_status_t spmm_plan_export(const int32_t *rowptr, const int32_t *colind,
                               int64_t M, int64_t K,
                               const spmm_tuning_t *resolved, void *stream_ptr,
                               int64_t cap, int64_t *counts,
                               int32_t *medium_rows, int32_t *long_rows,
                               int32_t *chunks, int32_t *hub_rows,
                               int32_t *hub_chunks)
{
    g_last_error.clear();
    if (resolved == nullptr || counts == nullptr)
        return fail(SPMM_ERROR_INVALID_VALUE, "null argument");
    if (resolved->short_max < 0 || resolved->medium_max < resolved->short_max ||
        resolved->chunk_nnz <= 0 || resolved->hub_min < 0 ||
        resolved->slab_rows <= 0 || resolved->reserved != 0)
        return fail(SPMM_ERROR_INVALID_VALUE, "tuning must be fully resolved");
    if (M < 0 || M >= kMaxIndex || K < 0 || K >= kMaxIndex || cap < 0)
        return fail(SPMM_ERROR_INVALID_VALUE, "M, K or cap out of range");
    if (cap > 0 && (medium_rows == nullptr || long_rows == nullptr || chunks == nullptr ||
                    hub_rows == nullptr || hub_chunks == nullptr))
        return fail(SPMM_ERROR_INVALID_VALUE, "null output array");
    for (int q = 0; q < 6; ++q)
        counts[q] = 0;
    if (M == 0)
        return SPMM_SUCCESS;
    if (rowptr == nullptr)
        return fail(SPMM_ERROR_INVALID_VALUE, "rowptr is null");
    if (colind == nullptr && resolved->hub_min < INT32_MAX)
        return fail(SPMM_ERROR_INVALID_VALUE, "colind is null (hub chunks need it)");

    hipStream_t stream = (hipStream_t)stream_ptr;
    const ScratchLayout lay = scratch_layout(M);
    const int64_t recs = cap > 0 ? cap : 1;
    char *dev_mem = nullptr;
    // scratch, then the exported arrays and counts
    const int64_t off_med = align_up(lay.total, 256);
    const int64_t off_long = align_up(off_med + 4 * recs, 256);
    const int64_t off_chunk = align_up(off_long + (int64_t)sizeof(LongRow) * recs, 256);
    const int64_t off_hub = align_up(off_chunk + (int64_t)sizeof(Chunk) * recs, 256);
    const int64_t off_hchunk = align_up(off_hub + 4 * recs, 256);
    const int64_t off_counts = align_up(off_hchunk + (int64_t)sizeof(Chunk) * recs, 256);
    const int64_t total = off_counts + 6 * 8;
    hipError_t err = hipMalloc(&dev_mem, (size_t)total);
    if (err != hipSuccess)
        return fail_hip(err, "hipMalloc");
    spmm_status_t st = SPMM_SUCCESS;
    do {
        if ((err = hipMemsetAsync(dev_mem, 0, (size_t)lay.total, stream)) != hipSuccess) {
            st = fail_hip(err, "hipMemsetAsync");
            break;
        }
        WorkerArgs wa;
        memset(&wa, 0, sizeof wa);
        wa.rowptr = rowptr;
        wa.colind = colind;
        wa.M = M;
        wa.K = K;
        wa.N = 1;
        wa.th = thresholds_of(*resolved, K);
        wa.plan = carve(dev_mem, lay);
        wa.shape = plan_shape(M);
        wa.epoch = 1;
        wa.wait_polls = current_wait_polls();
        wa.C = nullptr;  // plan only
        const WorkerConfig cfg = choose_worker(SPMM_DTYPE_F32, 1, nullptr, nullptr);
        int64_t dcounts[6];
        if ((err = launch_worker(cfg, wa, stream, nullptr, nullptr)) != hipSuccess ||
            (err = launch_plan_export(rowptr, colind, wa.th, wa.plan, 1, cap,
                                      (int32_t *)(dev_mem + off_med),
                                      (LongRow *)(dev_mem + off_long),
                                      (Chunk *)(dev_mem + off_chunk),
                                      (int32_t *)(dev_mem + off_hub),
                                      (Chunk *)(dev_mem + off_hchunk),
                                      (int64_t *)(dev_mem + off_counts), stream)) != hipSuccess ||
            (err = hipStreamSynchronize(stream)) != hipSuccess ||
            (err = hipMemcpy(dcounts, dev_mem + off_counts, sizeof dcounts,
                             hipMemcpyDeviceToHost)) != hipSuccess) {
            st = fail_hip(err, "plan");
            break;
        }
        for (int q = 0; q < 6; ++q)
            counts[q] = dcounts[q];
        const int64_t nm = dcounts[1] < cap ? dcounts[1] : cap;
        const int64_t nl = dcounts[2] < cap ? dcounts[2] : cap;
        const int64_t nc = dcounts[3] < cap ? dcounts[3] : cap;
        const int64_t nh = dcounts[4] < cap ? dcounts[4] : cap;
        const int64_t nhc = dcounts[5] < cap ? dcounts[5] : cap;
        if ((nm > 0 && (err = hipMemcpy(medium_rows, dev_mem + off_med, 4 * nm,
                                        hipMemcpyDeviceToHost)) != hipSuccess) ||
            (nl > 0 && (err = hipMemcpy(long_rows, dev_mem + off_long,
                                        sizeof(LongRow) * nl,
                                        hipMemcpyDeviceToHost)) != hipSuccess) ||
            (nc > 0 && (err = hipMemcpy(chunks, dev_mem + off_chunk,
                                        sizeof(Chunk) * nc,
                                        hipMemcpyDeviceToHost)) != hipSuccess) ||
            (nh > 0 && (err = hipMemcpy(hub_rows, dev_mem + off_hub, 4 * nh,
                                        hipMemcpyDeviceToHost)) != hipSuccess) ||
            (nhc > 0 && (err = hipMemcpy(hub_chunks, dev_mem + off_hchunk,
                                         sizeof(Chunk) * nhc,
                                         hipMemcpyDeviceToHost)) != hipSuccess)) {
            st = fail_hip(err, "copy plan");
            break;
        }
    } while (0);
    const hipError_t ferr = hipFree(dev_mem);
    if (st == SPMM_SUCCESS && ferr != hipSuccess)
        st = fail_hip(ferr, "hipFree");
    return st;
}

const char *spmm_status_string(spmm_status_t status)
{
    switch (status) {
    case SPMM_SUCCESS: return "SPMM_SUCCESS";
    case SPMM_ERROR_INVALID_VALUE: return "SPMM_ERROR_INVALID_VALUE";
    case SPMM_ERROR_HIP: return "SPMM_ERROR_HIP";
    case SPMM_ERROR_OUT_OF_MEMORY: return "SPMM_ERROR_OUT_OF_MEMORY";
    case SPMM_ERROR_UNSUPPORTED: return "SPMM_ERROR_UNSUPPORTED";
    default: return "SPMM_ERROR_UNKNOWN";
    }
}

const char *spmm_last_error(void) { return g_last_error.c_str(); }

spmm_status_t spmm_timing_enable(int32_t on)
{
    std::lock_guard<std::mutex> lock(g_time_mu);
    g_timing = on != 0;
    return SPMM_SUCCESS;
}

spmm_status_t spmm_timing_read(double *plan_ms, double *worker_ms,
                               int64_t *calls)
{
    g_last_error.clear();
    std::vector<TimedCall> taken;
    {
        std::lock_guard<std::mutex> lock(g_time_mu);
        taken.swap(g_timed);
    }
    double p = 0.0, w = 0.0;
    spmm_status_t st = SPMM_SUCCESS;
    for (const TimedCall &tc : taken) {
        float a = 0.0f, b = 0.0f;
        hipError_t err = hipEventSynchronize(tc.work1);
        if (err == hipSuccess)
            err = hipEventElapsedTime(&b, tc.work0, tc.work1);
        if (err != hipSuccess && st == SPMM_SUCCESS)
            st = fail_hip(err, "hipEventElapsedTime");
        p += a;
        w += b;
    }
    {
        std::lock_guard<std::mutex> lock(g_time_mu);
        for (const TimedCall &tc : taken) {
            g_free_events.push_back(tc.work0);
            g_free_events.push_back(tc.work1);
        }
    }
    if (plan_ms)
        *plan_ms = p;
    if (worker_ms)
        *worker_ms = w;
    if (calls)
        *calls = (int64_t)taken.size();
    return st;
}

spmm_status_t spmm_stream_release(void *stream_ptr)
{
    g_last_error.clear();
    hipStream_t stream = (hipStream_t)stream_ptr;
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess)
        return fail_hip(err, "hipGetDevice");
    StreamState *ss = stream_state(dev, stream, false);
    if (ss == nullptr)
        return SPMM_SUCCESS;  // never called on this stream
    std::lock_guard<std::mutex> guard(ss->mu);
    // stream-ordered frees after the calls already enqueued, then wait, so
    // that the stream can be destroyed and its handle reused safely
    if (ss->scratch && (err = hipFreeAsync(ss->scratch, stream)) != hipSuccess)
        return fail_hip(err, "hipFreeAsync");
    ss->scratch = nullptr;
    ss->scratch_size = 0;
    ss->epoch = 0;
    ss->faults_seen = 0;  // a new block starts its count at zero
    if (ss->aux && (err = hipFreeAsync(ss->aux, stream)) != hipSuccess)
        return fail_hip(err, "hipFreeAsync");
    ss->aux = nullptr;
    ss->aux_size = 0;
    if ((err = hipStreamSynchronize(stream)) != hipSuccess)
        return fail_hip(err, "hipStreamSynchronize");
    return SPMM_SUCCESS;
}

spmm_status_t spmm_stream_faults(void *stream_ptr, int64_t *faults)
{
    g_last_error.clear();
    if (faults == nullptr)
        return fail(SPMM_ERROR_INVALID_VALUE, "faults is null");
    *faults = 0;
    hipStream_t stream = (hipStream_t)stream_ptr;
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess)
        return fail_hip(err, "hipGetDevice");
    int64_t total = 0;
    uint32_t v = 0;
    StreamState *ss = stream_state(dev, stream, false);
    if (ss != nullptr) {
        std::lock_guard<std::mutex> guard(ss->mu);
        if (ss->scratch != nullptr) {  // else no block (yet, or released)
            if ((err = take_fault_count((char *)ss->scratch, stream, &ss->faults_seen, &v)) !=
                hipSuccess)
                return fail_hip(err, "reading the fault count");
            total += v;
        }
    }
    // the no-allocation calls' count, in this device's fixed array
    if (dev >= 0 && dev < kMaxDevices) {
        FixedScratch &fs = g_fixed[dev];
        std::lock_guard<std::mutex> guard(fs.mu);
        if (fs.ptr != nullptr) {
            if ((err = take_fault_count(fs.ptr, stream, &fs.faults_seen, &v)) != hipSuccess)
                return fail_hip(err, "reading the fixed array's fault count");
            total += v;
        }
    }
    *faults = total;
    return SPMM_SUCCESS;
}

spmm_status_t spmm_debug_set_wait_polls(int64_t polls)
{
    g_last_error.clear();
    if (polls > kWaitPolls)
        return fail(SPMM_ERROR_INVALID_VALUE,
                    "polls above the default bound " + std::to_string(kWaitPolls));
    g_wait_polls.store(polls < 0 ? kWaitPolls : (int32_t)polls, std::memory_order_relaxed);
    return SPMM_SUCCESS;
}

}  // extern "C"
