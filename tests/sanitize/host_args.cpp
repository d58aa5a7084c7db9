// Argument paths of the library's C ABI, run in a host-only build of the
// library sources under AddressSanitizer and UndefinedBehaviorSanitizer.
// Every call here is answered on the host (rejected, nothing to do, or a
// host-only query), so no GPU is needed; a sanitizer report, a wrong status
// or an empty error text ends the program with a non-zero status.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "spmm.h"

namespace {

int g_failures = 0;

void expect(bool ok, const char *what, int line)
{
    if (!ok) {
        std::fprintf(stderr, "line %d: %s (last error: \"%s\")\n", line, what,
                     spmm_last_error());
        ++g_failures;
    }
}

#define EXPECT(cond) expect((cond), #cond, __LINE__)

// An address that is never dereferenced: every call below returns before
// touching memory.
template <class T>
T *fake(uintptr_t offset = 0)
{
    return reinterpret_cast<T *>(uintptr_t{0x10000} + offset);
}

void status_strings()
{
    EXPECT(std::strcmp(spmm_status_string(SPMM_SUCCESS), "SPMM_SUCCESS") == 0);
    EXPECT(std::strcmp(spmm_status_string(SPMM_ERROR_UNSUPPORTED),
                       "SPMM_ERROR_UNSUPPORTED") == 0);
    EXPECT(std::strcmp(spmm_status_string(-5), "SPMM_ERROR_UNKNOWN") == 0);
}

void product_arguments()
{
    const int32_t *rp = fake<const int32_t>(), *ci = fake<const int32_t>();
    const float *v = fake<const float>(), *B = fake<const float>();
    float *C = fake<float>();
    struct Case {
        int64_t M, K, N;
        const int32_t *rowptr;
        const float *B;
        float *C;
        spmm_status_t want;
    } cases[] = {
        {-1, 4, 4, rp, B, C, SPMM_ERROR_INVALID_VALUE},
        {4, -1, 4, rp, B, C, SPMM_ERROR_INVALID_VALUE},
        {4, 4, -2, rp, B, C, SPMM_ERROR_INVALID_VALUE},
        {int64_t{1} << 31, 4, 4, rp, B, C, SPMM_ERROR_INVALID_VALUE},
        {4, int64_t{1} << 31, 4, rp, B, C, SPMM_ERROR_INVALID_VALUE},
        {INT64_MAX, INT64_MAX, INT64_MAX, rp, B, C, SPMM_ERROR_INVALID_VALUE},
        {4, 4, INT64_MAX, rp, B, C, SPMM_ERROR_INVALID_VALUE},
        {4, 4, 4, nullptr, B, C, SPMM_ERROR_INVALID_VALUE},
        {4, 4, 4, rp, nullptr, C, SPMM_ERROR_INVALID_VALUE},
        {4, 4, 4, rp, B, nullptr, SPMM_ERROR_INVALID_VALUE},
        {4, 4, 4, rp, B, fake<float>(2), SPMM_ERROR_INVALID_VALUE},
        {4, 4, 4, rp, fake<const float>(1), C, SPMM_ERROR_INVALID_VALUE},
        {0, 4, 4, nullptr, nullptr, nullptr, SPMM_SUCCESS},
        {4, 4, 0, nullptr, nullptr, nullptr, SPMM_SUCCESS},
    };
    for (const Case &c : cases) {
        const spmm_status_t st = spmm_csr_f32(c.rowptr, ci, v, c.B, c.C, c.M, c.K, c.N,
                                              nullptr);
        EXPECT(st == c.want);
        if (st != SPMM_SUCCESS)
            EXPECT(spmm_last_error()[0] != '\0');
    }
    // bf16 B needs 2-byte alignment only
    EXPECT(spmm_csr_bf16in_f32acc(rp, ci, fake<const uint16_t>(), fake<const uint16_t>(1), C,
                                  4, 4, 4, nullptr) == SPMM_ERROR_INVALID_VALUE);
    // tuned: bad order of thresholds, reserved field, unknown dtype
    spmm_tuning_t bad = {10, 5, 4, -1, 0, 0};
    EXPECT(spmm_csr_tuned(SPMM_DTYPE_F32, rp, ci, v, B, C, 4, 4, 4, &bad, nullptr) ==
           SPMM_ERROR_INVALID_VALUE);
    spmm_tuning_t reserved = {1, 5, 4, -1, 0, 1};
    EXPECT(spmm_csr_tuned(SPMM_DTYPE_F32, rp, ci, v, B, C, 4, 4, 4, &reserved, nullptr) ==
           SPMM_ERROR_INVALID_VALUE);
    EXPECT(spmm_csr_tuned(5, rp, ci, v, B, C, 4, 4, 4, nullptr, nullptr) ==
           SPMM_ERROR_INVALID_VALUE);
    // element-balanced kernel: the same checks
    EXPECT(spmm_csr_eb(SPMM_DTYPE_F32, rp, ci, v, B, C, -1, 4, 4, nullptr) ==
           SPMM_ERROR_INVALID_VALUE);
    EXPECT(spmm_csr_eb(SPMM_DTYPE_F32, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 4, 4,
                       nullptr) == SPMM_SUCCESS);
}

void noalloc_arguments()
{
    const int32_t *rp = fake<const int32_t>();
    // an M whose plan does not fit the fixed array: the message names the limit
    EXPECT(spmm_csr_tuned_noalloc(SPMM_DTYPE_F32, rp, rp, fake<const void>(),
                                  fake<const void>(), fake<float>(), int64_t{1} << 22, 4, 4,
                                  nullptr, nullptr) == SPMM_ERROR_UNSUPPORTED);
    EXPECT(std::strstr(spmm_last_error(), "at most") != nullptr);
    EXPECT(spmm_csr_tuned_noalloc(SPMM_DTYPE_F32, rp, rp, fake<const void>(),
                                  fake<const void>(), fake<float>(), -1, 4, 4, nullptr,
                                  nullptr) == SPMM_ERROR_INVALID_VALUE);
    EXPECT(spmm_csr_tuned_noalloc(SPMM_DTYPE_F32, nullptr, nullptr, nullptr, nullptr, nullptr,
                                  0, 4, 4, nullptr, nullptr) == SPMM_SUCCESS);
}

void resolve_tuning()
{
    const int64_t Ks[] = {0, 1, 1024, 262144, 1048576, (int64_t{1} << 31) - 1};
    const int64_t Ns[] = {1, 3, 32, 64, 256, 512, 1000, 4096, (int64_t{1} << 31) - 1};
    for (int dtype = 0; dtype < 2; ++dtype)
        for (int64_t K : Ks)
            for (int64_t N : Ns) {
                spmm_tuning_t t;
                EXPECT(spmm_resolve_tuning(dtype, K, N, nullptr, &t) == SPMM_SUCCESS);
                EXPECT(0 <= t.short_max && t.short_max <= t.medium_max);
                EXPECT(t.chunk_nnz > 0 && t.slab_rows > 0 && t.hub_min >= t.medium_max);
            }
    spmm_tuning_t req = {3, 77, 11, 5, 9, 0}, t;
    EXPECT(spmm_resolve_tuning(SPMM_DTYPE_F32, 100, 64, &req, &t) == SPMM_SUCCESS);
    EXPECT(t.short_max == 3 && t.medium_max == 77 && t.chunk_nnz == 11 && t.hub_min == 5 &&
           t.slab_rows == 9);
    spmm_tuning_t bad = {10, 5, 4, -1, 0, 0};
    EXPECT(spmm_resolve_tuning(SPMM_DTYPE_F32, 100, 64, &bad, &t) == SPMM_ERROR_INVALID_VALUE);
    EXPECT(spmm_resolve_tuning(7, 100, 64, nullptr, &t) == SPMM_ERROR_INVALID_VALUE);
    EXPECT(spmm_resolve_tuning(SPMM_DTYPE_F32, 100, -1, nullptr, &t) ==
           SPMM_ERROR_INVALID_VALUE);
    EXPECT(spmm_resolve_tuning(SPMM_DTYPE_F32, 100, 64, nullptr, nullptr) ==
           SPMM_ERROR_INVALID_VALUE);
}

void plan_export_arguments()
{
    int64_t counts[6];
    spmm_tuning_t unresolved = {-1, 5, 4, INT32_MAX, 1, 0};
    EXPECT(spmm_plan_export(fake<const int32_t>(), fake<const int32_t>(), 4, 4, &unresolved,
                            nullptr, 0, counts, nullptr, nullptr, nullptr, nullptr,
                            nullptr) == SPMM_ERROR_INVALID_VALUE);
    spmm_tuning_t hubs = {1, 5, 4, 10, 1, 0};
    EXPECT(spmm_plan_export(fake<const int32_t>(), nullptr, 4, 4, &hubs, nullptr, 0, counts,
                            nullptr, nullptr, nullptr, nullptr,
                            nullptr) == SPMM_ERROR_INVALID_VALUE);
    spmm_tuning_t none = {1, 5, 4, INT32_MAX, 1, 0};
    for (int64_t &c : counts)
        c = -7;
    EXPECT(spmm_plan_export(fake<const int32_t>(), nullptr, 0, 4, &none, nullptr, 0, counts,
                            nullptr, nullptr, nullptr, nullptr, nullptr) == SPMM_SUCCESS);
    for (int64_t c : counts)
        EXPECT(c == 0);
}

void sddmm_fusedmm_arguments()
{
    const int32_t *rp = fake<const int32_t>();
    const float *f = fake<const float>();
    float *o = fake<float>();
    EXPECT(sddmm_csr_f32(rp, rp, f, f, o, -1, 4, 4, 4, nullptr) == SPMM_ERROR_INVALID_VALUE);
    EXPECT(sddmm_csr_f32(rp, rp, f, f, o, 4, 4, 4, int64_t{1} << 31, nullptr) ==
           SPMM_ERROR_INVALID_VALUE);
    EXPECT(sddmm_csr_f32(rp, rp, f, f, o, 0, 4, 4, 3, nullptr) == SPMM_ERROR_INVALID_VALUE);
    EXPECT(sddmm_csr_f32(rp, rp, f, f, o, 4, 4, 0, 3, nullptr) == SPMM_ERROR_UNSUPPORTED);
    EXPECT(sddmm_csr_f32(rp, rp, f, f, fake<float>(1), 4, 4, 4, 3, nullptr) ==
           SPMM_ERROR_INVALID_VALUE);
    EXPECT(sddmm_csr_f32(nullptr, nullptr, nullptr, nullptr, nullptr, 4, 4, 4, 0, nullptr) ==
           SPMM_SUCCESS);
    EXPECT(sddmm_csr_bf16in_f32acc(rp, rp, fake<const uint16_t>(1), fake<const uint16_t>(),
                                   o, 4, 4, 4, 3, nullptr) == SPMM_ERROR_INVALID_VALUE);
    EXPECT(fusedmm_csr_f32(rp, rp, f, f, nullptr, o, 4, 4, 4, 3, nullptr) ==
           SPMM_ERROR_INVALID_VALUE);
    EXPECT(fusedmm_csr_f32(rp, rp, f, f, f, fake<float>(2), 4, 4, 4, 3, nullptr) ==
           SPMM_ERROR_INVALID_VALUE);
    EXPECT(fusedmm_csr_f32(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 4, 4, 0,
                           nullptr) == SPMM_SUCCESS);
    const uint16_t *h = fake<const uint16_t>();
    EXPECT(fusedmm_csr_bf16in_f32acc(rp, rp, h, h, nullptr, o, 4, 4, 12, 3, nullptr) ==
           SPMM_ERROR_INVALID_VALUE);
    EXPECT(fusedmm_csr_bf16in_f32acc(rp, rp, h, h, h, fake<float>(2), 4, 4, 1032, 3,
                                     nullptr) == SPMM_ERROR_INVALID_VALUE);
    EXPECT(fusedmm_csr_bf16in_f32acc(rp, rp, fake<const uint16_t>(1), h, h, o, 4, 4, 8, 3,
                                     nullptr) == SPMM_ERROR_INVALID_VALUE);
    const int64_t big = (int64_t{1} << 31) - 1;  // widened copy past 2^56 bytes
    EXPECT(fusedmm_csr_bf16in_f32acc(rp, rp, h, h, h, o, big, big, big, 3, nullptr) ==
           SPMM_ERROR_OUT_OF_MEMORY);
}

void hooks_and_timing()
{
    EXPECT(spmm_debug_set_wait_polls(int64_t{1} << 40) == SPMM_ERROR_INVALID_VALUE);
    EXPECT(spmm_debug_set_wait_polls(0) == SPMM_SUCCESS);
    EXPECT(spmm_debug_set_wait_polls(-1) == SPMM_SUCCESS);
    EXPECT(spmm_timing_enable(0) == SPMM_SUCCESS);
    double p = -1, w = -1;
    int64_t n = -1;
    EXPECT(spmm_timing_read(&p, &w, &n) == SPMM_SUCCESS);
    EXPECT(p == 0 && w == 0 && n == 0);
    int64_t faults = -1;
    EXPECT(spmm_stream_faults(nullptr, nullptr) == SPMM_ERROR_INVALID_VALUE);
    (void)faults;
}

}  // namespace

int main()
{
    status_strings();
    product_arguments();
    noalloc_arguments();
    resolve_tuning();
    plan_export_arguments();
    sddmm_fusedmm_arguments();
    hooks_and_timing();
    if (g_failures != 0) {
        std::fprintf(stderr, "%d check(s) failed\n", g_failures);
        return 1;
    }
    std::printf("host argument paths: ok\n");
    return 0;
}
