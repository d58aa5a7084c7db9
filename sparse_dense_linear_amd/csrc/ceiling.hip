// ceiling.hip -- measurement kernel (not part of the product path): the
// bandwidth this GPU reaches on the access pattern of a row-wise sparse x
// dense product stripped of everything else.  Output row i is the plain sum
// of D rows of B picked by idx[i*D .. i*D+D-1]: D random row gathers of
// N fp32 and one row store, with no plan, no values and no reduction across
// lanes.  bench.py --gather-ceiling times it to put the product's own
// bandwidth in context.
//
// Layout: B is K x N fp32 row-major, idx int32[M*D] (every entry in [0, K),
// a precondition), C is M x N fp32 row-major.  N is a multiple of 4 with
// N/4 a power of two in [4, 64]: a group of G = N/4 lanes covers a row with
// one 16-byte vector per lane, 64/G rows per wavefront.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int D>
__global__ __launch_bounds__(256) void gather_rows(const float *__restrict__ B,
                                                   const int32_t *__restrict__ idx,
                                                   float *__restrict__ C,
                                                   int64_t M, int64_t N, int G)
{
    const int lane = threadIdx.x & 63;
    const int g = lane / G, j = lane % G;
    const int64_t R = 64 / G;
    const int64_t wave = ((int64_t)blockIdx.x * 256 + threadIdx.x) / 64;
    const int64_t waves = (int64_t)gridDim.x * 4;
    for (int64_t r = wave * R + g; r < M; r += waves * R) {
        f32x4 v[D];
#pragma unroll
        for (int u = 0; u < D; ++u) {
            const int64_t col = idx[r * D + u];
            v[u] = *(const f32x4 *)(B + col * N + 4 * j);
        }
        f32x4 acc = v[0];
#pragma unroll
        for (int u = 1; u < D; ++u)
            acc += v[u];
        *(f32x4 *)(C + r * N + 4 * j) = acc;
    }
}

template <int D>
hipError_t launch(const float *B, const int32_t *idx, float *C, int64_t M,
                  int64_t N, hipStream_t s)
{
    const int G = (int)(N / 4);
    const int64_t R = 64 / G;
    int64_t blocks = (M + 4 * R - 1) / (4 * R);
    if (blocks > 8192)
        blocks = 8192;  // grid-stride beyond that
    hipLaunchKernelGGL(gather_rows<D>, dim3((unsigned)blocks), dim3(256), 0, s,
                       B, idx, C, M, N, G);
    return hipGetLastError();
}

}  // namespace

// Returns 0 on success, 1 for arguments outside the supported shapes, 2 for
// a HIP error.  Enqueued on `stream`; does not synchronise.
extern "C" int sdl_gather_ceiling(const float *B, const int32_t *idx, float *C,
                                  int64_t M, int64_t N, int32_t D, void *stream)
{
    if (B == nullptr || idx == nullptr || C == nullptr || M < 0)
        return 1;
    if (N % 4 != 0 || N / 4 < 4 || N / 4 > 64 || ((N / 4) & (N / 4 - 1)) != 0)
        return 1;
    if ((((uintptr_t)B) | ((uintptr_t)C)) % 16 != 0)
        return 1;
    if (M == 0)
        return 0;
    hipStream_t s = (hipStream_t)stream;
    hipError_t err;
    switch (D) {
    case 1: err = launch<1>(B, idx, C, M, N, s); break;
    case 2: err = launch<2>(B, idx, C, M, N, s); break;
    case 4: err = launch<4>(B, idx, C, M, N, s); break;
    case 8: err = launch<8>(B, idx, C, M, N, s); break;
    case 16: err = launch<16>(B, idx, C, M, N, s); break;
    default: return 1;
    }
    return err == hipSuccess ? 0 : 2;
}
