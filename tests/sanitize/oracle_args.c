/*
 * The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer: every
 * array is allocated at its exact size, so a read or write one element past
 * any of them is reported.  Inputs are small integers (exact in fp32, bf16
 * and fp64), so each result is compared exactly with a dense brute-force
 * computation written here; bad arguments must return -1.  A sanitizer
 * report or a wrong value ends the program with a non-zero status.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_spmm(int64_t M, int64_t N, const int32_t *rowptr, const int32_t *colind,
                int val_kind, const void *vals, int b_kind, const void *B,
                const int64_t *rows, int64_t nrows, double *C_out, double *S_out);
int oracle_sddmm(int64_t M, int64_t N, const int32_t *rowptr, const int32_t *colind,
                 int kind, const void *C, const void *B, const int64_t *rows,
                 int64_t nrows, int64_t *out_off, double *A_out, double *S_out);
int oracle_fusedmm(int64_t M, int64_t N, const int32_t *rowptr, const int32_t *colind,
                   int kind, const void *C, const void *B, const void *D,
                   const int64_t *rows, int64_t nrows, double *E_out, double *T_out);

static int failures = 0;
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "line %d: %s\n", __LINE__, #c); ++failures; } } while (0)

/* bf16 bit pattern of a small integer (exact: the upper half of its fp32). */
static uint16_t bf16_of(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    return (uint16_t)(u >> 16);
}

enum { M = 7, K = 5, N = 3, OFF = 2 };
/* rows: 0 empty, 1 one entry, 2 a repeated column, 3 empty, 4 all columns,
 * 5 one entry, 6 empty (the last row) */
static const int32_t lens[M] = {0, 1, 3, 0, 5, 1, 0};
static const int32_t cols[] = {4, 1, 1, 3, 0, 1, 2, 3, 4, 2};

static void *exact(size_t bytes) { return malloc(bytes ? bytes : 1); }

int main(void)
{
    int32_t *rowptr = exact((M + 1) * sizeof(int32_t));
    int64_t nnz = 0, i, n, p, r;
    rowptr[0] = OFF;
    for (i = 0; i < M; ++i)
        rowptr[i + 1] = rowptr[i] + lens[i];
    nnz = rowptr[M] - OFF;
    int32_t *colind = exact((size_t)(OFF + nnz) * sizeof(int32_t));
    float *vals = exact((size_t)(OFF + nnz) * sizeof(float));
    uint16_t *vals16 = exact((size_t)(OFF + nnz) * sizeof(uint16_t));
    float *B = exact(K * N * sizeof(float)), *Cd = exact(M * N * sizeof(float));
    float *D = exact(K * N * sizeof(float));
    uint16_t *B16 = exact(K * N * sizeof(uint16_t));
    for (p = 0; p < OFF; ++p) {
        colind[p] = 0;
        vals[p] = 0.0f;
        vals16[p] = 0;
    }
    for (p = 0; p < nnz; ++p) {
        colind[OFF + p] = cols[p];
        vals[OFF + p] = (float)((p % 5) - 2);      /* -2 .. 2 */
        vals16[OFF + p] = bf16_of(vals[OFF + p]);
    }
    for (i = 0; i < K * N; ++i) {
        B[i] = (float)((i * 7) % 9 - 4);
        B16[i] = bf16_of(B[i]);
        D[i] = (float)((i * 5) % 7 - 3);
    }
    for (i = 0; i < M * N; ++i)
        Cd[i] = (float)((i * 3) % 5 - 2);

    /* SpMM, every row, both element kinds: dense brute force */
    double *want = exact(M * N * sizeof(double)), *bound = exact(M * N * sizeof(double));
    for (i = 0; i < M; ++i)
        for (n = 0; n < N; ++n) {
            double a = 0, s = 0;
            for (p = rowptr[i]; p < rowptr[i + 1]; ++p) {
                a += (double)vals[p] * B[colind[p] * N + n];
                s += abs((int)vals[p]) * abs((int)B[colind[p] * N + n]);
            }
            want[i * N + n] = a;
            bound[i * N + n] = s;
        }
    double *C_out = exact(M * N * sizeof(double)), *S_out = exact(M * N * sizeof(double));
    for (int kind = 0; kind < 2; ++kind) {
        CHECK(oracle_spmm(M, N, rowptr, colind, kind, kind ? (void *)vals16 : (void *)vals,
                          kind, kind ? (void *)B16 : (void *)B, NULL, 0, C_out, S_out) == 0);
        for (i = 0; i < M * N; ++i)
            CHECK(C_out[i] == want[i] && S_out[i] == bound[i]);
    }
    /* a sample of rows, in any order, without the bound */
    const int64_t pick[3] = {6, 2, 4};
    double *C3 = exact(3 * N * sizeof(double));
    CHECK(oracle_spmm(M, N, rowptr, colind, 0, vals, 0, B, pick, 3, C3, NULL) == 0);
    for (r = 0; r < 3; ++r)
        for (n = 0; n < N; ++n)
            CHECK(C3[r * N + n] == want[pick[r] * N + n]);
    /* bad arguments */
    const int64_t outside[1] = {M};
    CHECK(oracle_spmm(M, N, rowptr, colind, 0, vals, 0, B, outside, 1, C3, NULL) == -1);
    CHECK(oracle_spmm(-1, N, rowptr, colind, 0, vals, 0, B, NULL, 0, C_out, NULL) == -1);
    CHECK(oracle_spmm(M, N, rowptr, colind, 2, vals, 0, B, NULL, 0, C_out, NULL) == -1);
    CHECK(oracle_spmm(0, N, rowptr, colind, 0, vals, 0, B, NULL, 0, C_out, NULL) == 0);

    /* SDDMM: A[p] = <C_i, B_j>; FusedMM: E_i = sum_p A[p] * D_j */
    double *A_out = exact((size_t)nnz * sizeof(double)), *AS = exact((size_t)nnz * sizeof(double));
    CHECK(oracle_sddmm(M, N, rowptr, colind, 0, Cd, B, NULL, 0, NULL, A_out, AS) == 0);
    double *E_out = exact(M * N * sizeof(double)), *T_out = exact(M * N * sizeof(double));
    CHECK(oracle_fusedmm(M, N, rowptr, colind, 0, Cd, B, D, NULL, 0, E_out, T_out) == 0);
    for (i = 0; i < M; ++i) {
        double e[N] = {0};
        for (p = rowptr[i]; p < rowptr[i + 1]; ++p) {
            double dot = 0;
            for (n = 0; n < N; ++n)
                dot += (double)Cd[i * N + n] * B[colind[p] * N + n];
            CHECK(A_out[p - OFF] == dot);
            for (n = 0; n < N; ++n)
                e[n] += dot * D[colind[p] * N + n];
        }
        for (n = 0; n < N; ++n)
            CHECK(E_out[i * N + n] == e[n]);
    }
    /* SDDMM of listed rows, packed in list order */
    int64_t off[3];
    double *A3 = exact((size_t)(lens[6] + lens[2] + lens[4]) * sizeof(double));
    CHECK(oracle_sddmm(M, N, rowptr, colind, 0, Cd, B, pick, 3, off, A3, NULL) == 0);
    CHECK(off[0] == 0 && off[1] == 0 && off[2] == lens[2]);
    for (r = 0; r < 3; ++r)
        for (p = 0; p < lens[pick[r]]; ++p)
            CHECK(A3[off[r] + p] == A_out[rowptr[pick[r]] - OFF + p]);
    CHECK(oracle_sddmm(M, N, rowptr, colind, 0, Cd, B, outside, 1, off, A3, NULL) == -1);
    CHECK(oracle_sddmm(M, N, rowptr, colind, 0, Cd, B, pick, 3, NULL, A3, NULL) == -1);
    CHECK(oracle_fusedmm(M, N, rowptr, colind, 0, Cd, B, D, outside, 1, E_out, NULL) == -1);
    CHECK(oracle_fusedmm(M, -1, rowptr, colind, 0, Cd, B, D, NULL, 0, E_out, NULL) == -1);

    free(rowptr); free(colind); free(vals); free(vals16); free(B); free(Cd); free(D);
    free(B16); free(want); free(bound); free(C_out); free(S_out); free(C3); free(A_out);
    free(AS); free(E_out); free(T_out); free(A3);
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle argument paths: ok\n");
    return 0;
}
