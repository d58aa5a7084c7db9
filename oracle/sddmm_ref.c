/*
 * sddmm_ref.c -- plain fp64 CPU oracle for the sampled dense-dense product
 * (SDDMM) and for its fusion with the sparse x dense product (FusedMM).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path loads, links or
 * calls this file; only the tests and the benchmark's CPU-baseline leg do.
 * It shares no source with the HIP library.
 *
 * Page cited throughout:
 *   [IntelMax] "Performance Optimization of Deep Learning Sparse Matrix
 *              Kernels on Intel Max Series GPU".
 *
 * SDDMM ([IntelMax], the SDDMM operation: Fig. 3 and Algorithm 1).  The
 * sparsity pattern of A is given in CSR form (rowptr = "ia", colind = "ja");
 * C is dense M x N and B is dense K x N, both row-major.  The value of the
 * stored entry p of row i, at column j = colind[p], is the dot product of
 * row C_i with column j of B^T, i.e. with row B_j:
 *     A[p] = sum over n of C[i][n] * B[j][n].
 * The entries of row i are computed in CSR order; each dot product sums n
 * upwards.  Reading taken (the equation is missing from the page): the
 * result replaces the values of A; it is not scaled by them.
 *
 * FusedMM ([IntelMax], the FusedMM operation: Fig. 6 and Algorithm 3).
 * The row of SDDMM values is not stored but used at once as the values of
 * a sparse x dense product with a third dense matrix D (K x N, row-major):
 *     E_i = sum over the entries p of row i of A[p] * D_{colind[p]},
 * with A[p] the SDDMM value above.  Reading taken: D has the same number of
 * columns N as C and B (the page uses one row length for every dense row),
 * and E starts from zero.
 *
 * Bounds returned with the results scale every tolerance:
 *   S[p]    = sum over n of |C[i][n]| * |B[j][n]|             (SDDMM)
 *   T[i][n] = sum over p of S[p] * |D[colind[p]][n]|          (FusedMM)
 *
 * Arithmetic: IEEE double in the page's order; compile with
 * -ffp-contract=off.  bf16 inputs are widened exactly (the 16 stored bits
 * are the high half of a binary32 word).  The only parallelism is an
 * OpenMP loop over independent rows.
 */
#include <stdint.h>
#include <string.h>
#include <math.h>

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };

static double widen_bf16(uint16_t bits)
{
    uint32_t word = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &word, sizeof f);
    return (double)f;
}

static double load_elem(const void *base, int kind, int64_t idx)
{
    if (kind == ORACLE_BF16)
        return widen_bf16(((const uint16_t *)base)[idx]);
    return (double)((const float *)base)[idx];
}

/* [IntelMax] Algorithm 1, one entry: row C_i times row B_j (column j of
 * B^T), summed over n upwards.  *bound receives sum |C_i[n]| |B_j[n]|. */
static double dot_entry(int64_t i, int64_t j, int64_t N, int kind,
                        const void *C, const void *B, double *bound)
{
    double acc = 0.0, s = 0.0;
    int64_t n;
    for (n = 0; n < N; ++n) {
        double c = load_elem(C, kind, i * N + n);
        double b = load_elem(B, kind, j * N + n);
        acc = acc + c * b;
        s = s + fabs(c) * fabs(b);
    }
    *bound = s;
    return acc;
}

/* Where the listed rows' entries start in the packed output: out_off[r]
 * for the r-th listed row, and the total.  Returns -1 on a bad row id. */
static int64_t packed_offsets(int64_t M, const int32_t *rowptr,
                              const int64_t *rows, int64_t nrows,
                              int64_t *out_off)
{
    int64_t r, total = 0;
    for (r = 0; r < nrows; ++r) {
        int64_t i = rows[r];
        if (i < 0 || i >= M)
            return -1;
        out_off[r] = total;
        total += (int64_t)rowptr[i + 1] - rowptr[i];
    }
    return total;
}

/*
 * SDDMM values (and bounds when S_out is not NULL).
 *   rows == NULL : every row; entry p goes to A_out[p - rowptr[0]]
 *   rows != NULL : the listed rows, their entries packed in list order
 *                  (row r's entries start at the sum of the lengths of the
 *                  rows listed before it); out_off (nrows int64, scratch
 *                  supplied by the caller) receives those starts
 * Returns 0, or -1 on a bad argument.
 */
int oracle_sddmm(int64_t M, int64_t N, const int32_t *rowptr,
                 const int32_t *colind, int kind, const void *C,
                 const void *B, const int64_t *rows, int64_t nrows,
                 int64_t *out_off, double *A_out, double *S_out)
{
    int64_t r, count;
    if (M < 0 || N < 0 || (kind != ORACLE_F32 && kind != ORACLE_BF16))
        return -1;
    if (rows != NULL) {
        if (out_off == NULL || packed_offsets(M, rowptr, rows, nrows, out_off) < 0)
            return -1;
        count = nrows;
    } else {
        count = M;
    }
#pragma omp parallel for schedule(dynamic, 64)
    for (r = 0; r < count; ++r) {
        int64_t i = rows ? rows[r] : r;
        int64_t base = rows ? out_off[r] : (int64_t)rowptr[i] - rowptr[0];
        int64_t p;
        for (p = rowptr[i]; p < rowptr[i + 1]; ++p) {
            double bound;
            int64_t o = base + (p - rowptr[i]);
            A_out[o] = dot_entry(i, colind[p], N, kind, C, B, &bound);
            if (S_out)
                S_out[o] = bound;
        }
    }
    return 0;
}

/*
 * FusedMM rows of E (and of the bound T when T_out is not NULL), [IntelMax]
 * Algorithm 3: for each entry of row i in CSR order, its SDDMM value a is
 * computed and a * D_{colind[p]} is added into the accumulator row.
 *   rows == NULL : every row, written to E_out[i*N + n]
 *   rows != NULL : the listed rows, written to E_out[r*N + n]
 * The output rows themselves are the accumulators.
 * Returns 0, or -1 on a bad argument.
 */
int oracle_fusedmm(int64_t M, int64_t N, const int32_t *rowptr,
                   const int32_t *colind, int kind, const void *C,
                   const void *B, const void *D, const int64_t *rows,
                   int64_t nrows, double *E_out, double *T_out)
{
    int64_t r, count;
    if (M < 0 || N < 0 || (kind != ORACLE_F32 && kind != ORACLE_BF16))
        return -1;
    if (rows != NULL) {
        for (r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= M)
                return -1;
        count = nrows;
    } else {
        count = M;
    }
#pragma omp parallel for schedule(dynamic, 64)
    for (r = 0; r < count; ++r) {
        int64_t i = rows ? rows[r] : r;
        double *e = E_out + r * N;
        double *t = T_out ? T_out + r * N : NULL;
        int64_t n, p;
        for (n = 0; n < N; ++n) {
            e[n] = 0.0;
            if (t)
                t[n] = 0.0;
        }
        for (p = rowptr[i]; p < rowptr[i + 1]; ++p) {
            int64_t j = colind[p];
            double bound;
            double a = dot_entry(i, j, N, kind, C, B, &bound);   /* SDDMM value */
            for (n = 0; n < N; ++n) {
                double d = load_elem(D, kind, j * N + n);
                e[n] = e[n] + a * d;                            /* E_i += a * D_j */
                if (t)
                    t[n] = t[n] + bound * fabs(d);
            }
        }
    }
    return 0;
}
