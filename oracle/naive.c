/*
 * CPU oracle, plain C, float64: BaKron-naive.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link or call this
 * file; only the tests, the smoke check and the bench's CPU-baseline leg do.
 * It shares no code with the GPU library.
 *
 * Follows "BaKron: Efficient Quantization with Kronecker-Factored Hessians"
 * (arXiv 2608.06291), §3.2, Algorithm 2 (GPTQ run on vec(W) with the Hessian
 * A (x) B): visit the entries one at a time in an order that respects
 * (i,j) <= (p,q) iff i<=p and j<=q; round the current entry; add the error
 * times the outer product of column i of the normalised factor of B and
 * column j of the normalised factor of A to the whole matrix. The visiting
 * order is the column-major vec order of §3.1 by default (order=0); order=1
 * is the row-major loop the printed algorithm uses. Appendix B shows both
 * give the same codes in exact arithmetic.
 *
 * "round" is replaced by the quantizer of §3.1: the closest element of the
 * alphabet after dividing by the scale of the entry's row or column.
 * Ties are broken to even (rint in the default rounding mode); the pages
 * only say a tie rule is fixed (Appendix B).
 *
 * Build: gcc -O2 -fPIC -shared -ffp-contract=off (see oracle/build.py).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

static double quantize_code(double x, double s, double lo, double hi, int unbounded)
{
    double c = rint(x / s);
    if (!unbounded) {
        if (c < lo) c = lo;
        if (c > hi) c = hi;
    }
    return c;
}

/*
 * W      m x n row-major (leading dim ldw), updated in place (it ends holding
 *        the quantised values s*c, as Algorithm 2 does).
 * LA     n x n unit-lower normalised factor of A, row-major (ldla).
 * LB     m x m unit-lower normalised factor of B, row-major (ldlb).
 * srow   per-row scales (length m) or NULL; scol per-column scales or NULL.
 *        Both NULL means s = 1.
 * forced m x n codes to impose instead of rounding (NULL = round freely);
 *        used to re-run the recursion with given codes.
 * C      out: codes (exact integers held as doubles), m x n (ldc).
 * Wt     out: the value each entry had when it was rounded (ldwt).
 * E      out: error s*c - Wt for each entry (lde).
 * order  0 = column-major vec order, 1 = row-major order.
 */
int bk_oracle_naive(int64_t m, int64_t n,
                    double *W, int64_t ldw,
                    const double *LA, int64_t ldla,
                    const double *LB, int64_t ldlb,
                    const double *srow, const double *scol,
                    double lo, double hi, int unbounded,
                    const double *forced, int64_t ldf,
                    double *C, int64_t ldc,
                    double *Wt, int64_t ldwt,
                    double *E, int64_t lde,
                    int order)
{
    if (m < 0 || n < 0) return -1;
    int64_t total = m * n;
    for (int64_t t = 0; t < total; ++t) {
        int64_t i, j;
        if (order == 0) { j = t / (m ? m : 1); i = t - j * m; }
        else            { i = t / (n ? n : 1); j = t - i * n; }
        double s = 1.0;
        if (srow) s = srow[i];
        else if (scol) s = scol[j];
        double x = W[i * ldw + j];
        double c = forced ? forced[i * ldf + j] : quantize_code(x, s, lo, hi, unbounded);
        double e = s * c - x;
        C[i * ldc + j] = c;
        Wt[i * ldwt + j] = x;
        E[i * lde + j] = e;
        /* W <- W + LB_i * e * (LA_j)^T, restricted to where the factors are
         * structurally non-zero (rows p >= i, columns q >= j). */
        for (int64_t p = i; p < m; ++p) {
            double bp = LB[p * ldlb + i] * e;
            if (bp == 0.0) continue;
            double *wrow = W + p * ldw;
            for (int64_t q = j; q < n; ++q)
                wrow[q] += bp * LA[q * ldla + j];
        }
    }
    return 0;
}
