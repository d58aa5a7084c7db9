/*
 * spmm_ref.c -- plain fp64 CPU oracle for CSR sparse x dense products.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path loads, links or
 * calls this file; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark do.  It shares no source with the HIP library.
 *
 * Page cited throughout:
 *   [IntelMax] "Performance Optimization of Deep Learning Sparse Matrix
 *              Kernels on Intel Max Series GPU".
 *
 * What is computed ([IntelMax], the SpMM operation: Fig. 5 and Algorithm 2):
 * the dense M x N result C = A * B, with A sparse in CSR form
 * (rowptr = "ia", colind = "ja", vals = "avalues") and B dense K x N,
 * row-major.  Row C_i is built by walking the stored non-zeros of row i in
 * their CSR order: for each one, the scalar s (the stored value) and its
 * column index k are fetched, and s times row B_k is added to C_i -- a SAXPY
 * over the N entries of the row.  C_i starts from zero (the page computes C,
 * it does not update it), so rows with no stored entries are zero rows.
 *
 * Readings taken where the page is silent (all listed in the design notes):
 *   - every stored entry is visited, so duplicate (i, k) entries are summed;
 *   - rowptr holds absolute offsets into colind/vals; rowptr[0] need not be 0;
 *   - bf16 inputs are widened exactly: the 16 stored bits become the high
 *     half of an IEEE binary32 word, which is then converted to double.
 *
 * Arithmetic: every product and sum is carried in IEEE double, in the
 * page's order (ascending position p inside the row).  The file must be
 * compiled with -ffp-contract=off so that no fused multiply-add changes the
 * rounding of a*b + acc.
 *
 * Besides C the oracle returns S, the element-wise bound
 *   S[i][n] = sum over the entries p of row i of |vals[p]| * |B[colind[p]][n]|,
 * which scales the tolerance of every floating-point comparison.
 *
 * The only parallelism is an OpenMP loop over independent rows; each row is
 * computed by one thread in the sequential order above, so the result does
 * not depend on the thread count.
 */
#include <stdint.h>
#include <string.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };

/* bf16 -> double, exact: bf16 is the upper half of a binary32 word. */
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

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of later calls' row loop (n >= 1); the arithmetic of a row does
 * not depend on it.  Used to time the oracle on one core. */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/*
 * One output row, [IntelMax] Algorithm 2: loop over the non-zeros of row i;
 * fetch the value s and the column k; add s * B_k into the accumulator row.
 * acc and bound (if not NULL) receive N doubles each.
 */
static void one_row(int64_t i, int64_t N,
                    const int32_t *rowptr, const int32_t *colind,
                    int val_kind, const void *vals,
                    int b_kind, const void *B,
                    double *acc, double *bound)
{
    int64_t n, p;
    for (n = 0; n < N; ++n) {
        acc[n] = 0.0;
        if (bound)
            bound[n] = 0.0;
    }
    for (p = rowptr[i]; p < rowptr[i + 1]; ++p) {
        double s = load_elem(vals, val_kind, p);   /* value of the entry */
        int64_t k = colind[p];                     /* its column index   */
        const int64_t brow = k * N;                /* start of row B_k   */
        for (n = 0; n < N; ++n) {
            double b = load_elem(B, b_kind, brow + n);
            acc[n] = acc[n] + s * b;               /* SAXPY: C_i += s*B_k */
            if (bound)
                bound[n] = bound[n] + fabs(s) * fabs(b);
        }
    }
}

/*
 * Compute rows of C (and of S when S_out is not NULL).
 *
 *   rows == NULL : all rows 0..M-1, written to C_out[i*N + n]
 *   rows != NULL : the nrows listed rows, written to C_out[r*N + n] for the
 *                  r-th listed row (a sample of a large problem)
 *
 * Returns 0 on success, -1 on a bad argument (a listed row outside [0, M),
 * negative sizes, unknown element kind).  The CSR arrays themselves are
 * trusted: the caller passes well-formed rowptr/colind.
 */
int oracle_spmm(int64_t M, int64_t N,
                const int32_t *rowptr, const int32_t *colind,
                int val_kind, const void *vals,
                int b_kind, const void *B,
                const int64_t *rows, int64_t nrows,
                double *C_out, double *S_out)
{
    int64_t r, count;
    int bad = 0;
    if (M < 0 || N < 0 || nrows < 0)
        return -1;
    if ((val_kind != ORACLE_F32 && val_kind != ORACLE_BF16) ||
        (b_kind != ORACLE_F32 && b_kind != ORACLE_BF16))
        return -1;
    count = rows ? nrows : M;
    if (rows) {
        for (r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= M)
                bad = 1;
        if (bad)
            return -1;
    }
#pragma omp parallel for schedule(dynamic, 16)
    for (r = 0; r < count; ++r) {
        int64_t i = rows ? rows[r] : r;
        one_row(i, N, rowptr, colind, val_kind, vals, b_kind, B,
                C_out + r * N, S_out ? S_out + r * N : (double *)0);
    }
    return 0;
}
