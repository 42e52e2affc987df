/*
 * oracle.c -- plain fp64 CPU reference of the block-sparse linear layer.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. The product path never
 * calls it, and it shares no code, header or table with the HIP library.
 *
 * What is computed (pytorch/ao sparsity README, workflow section: sparse and
 * dense matmul with the zero-filled weight are numerically equivalent; Table
 * 4.1: BSR stores dense blocks plus their block coordinates, CSR/CSC store an
 * index pointer, indices and data):
 *
 *   W~ [N,K] is zero except block (r, col_idx[i]) = V[i] for i in
 *   row_ptr[r] .. row_ptr[r+1]-1, with V[i][p][q] = W~[r*b+p][col_idx[i]*b+q].
 *
 *   forward       Y  = X . W~^T + 1 . bias^T                 (nn.Linear layout)
 *   input grad    dX = dY . W~
 *   weight grad   dV[i] = block (r, col_idx[i]) of dY^T . X  (the dense weight
 *                 gradient masked to the pattern, "dW' = dW (Mask)" of the
 *                 README's out-of-place mask update)
 *   bias grad     db = sum over rows of dY
 *
 * Alongside every output element o the oracle returns S(o), the sum of the
 * absolute values of the products summed into o (plus |bias| where a bias is
 * added). The tolerance of a bf16 result g is |g - o| <= 4e-3 * S(o).
 *
 * Every sum runs in a fixed order (stated per function), so the result does
 * not depend on the OpenMP thread count: threads only split independent
 * outputs (rows m, or blocks i).
 *
 * All matrices are dense row-major fp64. M is the number of rows of X / dY.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Forward. For each output Y[m][r*b+p]: sum over the blocks i of row r in
 * ascending i, then over q ascending, of X[m][col_idx[i]*b+q] * V[i][p][q];
 * then + bias. Empty block rows give bias (or 0). S may be NULL. */
void oracle_fwd(int64_t M, int32_t N, int32_t K, int32_t b,
                const int32_t *row_ptr, const int32_t *col_idx,
                const double *X, const double *V, const double *bias,
                double *Y, double *S)
{
    const int32_t R = N / b;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        const double *x = X + m * (int64_t)K;
        for (int32_t r = 0; r < R; ++r) {
            for (int32_t p = 0; p < b; ++p) {
                double acc = 0.0, s = 0.0;
                for (int32_t i = row_ptr[r]; i < row_ptr[r + 1]; ++i) {
                    const double *v = V + ((int64_t)i * b + p) * b;
                    const double *xc = x + (int64_t)col_idx[i] * b;
                    for (int32_t q = 0; q < b; ++q) {
                        double t = xc[q] * v[q];
                        acc += t;
                        s += fabs(t);
                    }
                }
                const int64_t n = (int64_t)r * b + p;
                if (bias) {
                    acc += bias[n];
                    s += fabs(bias[n]);
                }
                Y[m * (int64_t)N + n] = acc;
                if (S) S[m * (int64_t)N + n] = s;
            }
        }
    }
}

/* Input gradient, walking the CSR order on purpose (not the transposed
 * metadata): dX[m][col_idx[i]*b+q] += dY[m][r*b+p] * V[i][p][q] over rows r
 * ascending, blocks i ascending, p ascending. Columns of dX that no block
 * touches stay 0. S may be NULL. */
void oracle_dx(int64_t M, int32_t N, int32_t K, int32_t b,
               const int32_t *row_ptr, const int32_t *col_idx,
               const double *dY, const double *V,
               double *dX, double *S)
{
    const int32_t R = N / b;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        const double *dy = dY + m * (int64_t)N;
        double *dx = dX + m * (int64_t)K;
        double *s = S ? S + m * (int64_t)K : NULL;
        for (int32_t k = 0; k < K; ++k) {
            dx[k] = 0.0;
            if (s) s[k] = 0.0;
        }
        for (int32_t r = 0; r < R; ++r) {
            for (int32_t i = row_ptr[r]; i < row_ptr[r + 1]; ++i) {
                const int64_t c0 = (int64_t)col_idx[i] * b;
                for (int32_t p = 0; p < b; ++p) {
                    const double g = dy[(int64_t)r * b + p];
                    const double *v = V + ((int64_t)i * b + p) * b;
                    for (int32_t q = 0; q < b; ++q) {
                        double t = g * v[q];
                        dx[c0 + q] += t;
                        if (s) s[c0 + q] += fabs(t);
                    }
                }
            }
        }
    }
}

/* Weight gradient on the pattern only. For block i of row r, column c:
 * dV[i][p][q] = sum over m ascending of dY[m][r*b+p] * X[m][c*b+q].
 * `blocks` lists which block indices to compute (NULL = all nnzb, in order);
 * output slot j of dV (and S) holds block blocks[j]. */
void oracle_dw(int64_t M, int32_t N, int32_t K, int32_t b,
               const int32_t *row_ptr, const int32_t *col_idx,
               const double *dY, const double *X,
               const int32_t *blocks, int32_t nblocks,
               double *dV, double *S)
{
    const int32_t R = N / b;
    const int32_t nnzb = row_ptr[R];
    if (!blocks) nblocks = nnzb;
    /* row of every block, from the row pointer */
    int32_t *row_of = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nnzb > 0 ? nnzb : 1));
    for (int32_t r = 0; r < R; ++r)
        for (int32_t i = row_ptr[r]; i < row_ptr[r + 1]; ++i) row_of[i] = r;

#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t j = 0; j < nblocks; ++j) {
        const int32_t i = blocks ? blocks[j] : j;
        const int64_t n0 = (int64_t)row_of[i] * b;
        const int64_t k0 = (int64_t)col_idx[i] * b;
        double *acc = dV + (int64_t)j * b * b;
        double *s = S ? S + (int64_t)j * b * b : NULL;
        for (int32_t e = 0; e < b * b; ++e) {
            acc[e] = 0.0;
            if (s) s[e] = 0.0;
        }
        for (int64_t m = 0; m < M; ++m) {
            const double *dy = dY + m * (int64_t)N + n0;
            const double *x = X + m * (int64_t)K + k0;
            for (int32_t p = 0; p < b; ++p) {
                for (int32_t q = 0; q < b; ++q) {
                    double t = dy[p] * x[q];
                    acc[p * b + q] += t;
                    if (s) s[p * b + q] += fabs(t);
                }
            }
        }
    }
    free(row_of);
}

/* Bias gradient: db[n] = sum over m ascending of dY[m][n]; S = sum |dY|. */
void oracle_db(int64_t M, int32_t N, const double *dY, double *db, double *S)
{
#pragma omp parallel for schedule(static)
    for (int32_t n = 0; n < N; ++n) {
        double acc = 0.0, s = 0.0;
        for (int64_t m = 0; m < M; ++m) {
            acc += dY[m * (int64_t)N + n];
            s += fabs(dY[m * (int64_t)N + n]);
        }
        db[n] = acc;
        if (S) S[n] = s;
    }
}

/* Block magnitudes of a dense weight W [N][K] (pytorch/ao sparsity README,
 * Table 4.2: the magnitude criterion removes the parameters with the lowest
 * norm, L1 being the usual one; the criteria list's "weights" option scores
 * with the weight tensor alone). For block (r, c):
 *   norm = sum over p ascending of ( sum over q ascending of t(W[r*b+p][c*b+q]) )
 * with t(w) = |w| (kind 1, L1) or w*w (kind 2, squared L2), every sum taken
 * left to right in fp64 starting from 0. norms is [N/b][K/b] row-major. */
void oracle_block_norms(int32_t N, int32_t K, int32_t b, int32_t kind,
                        const double *W, double *norms)
{
    const int32_t R = N / b, C = K / b;
#pragma omp parallel for schedule(static)
    for (int32_t r = 0; r < R; ++r) {
        for (int32_t c = 0; c < C; ++c) {
            double acc = 0.0;
            for (int32_t p = 0; p < b; ++p) {
                const double *w = W + ((int64_t)r * b + p) * K + (int64_t)c * b;
                double row = 0.0;
                for (int32_t q = 0; q < b; ++q)
                    row += kind == 1 ? fabs(w[q]) : w[q] * w[q];
                acc += row;
            }
            norms[(int64_t)r * C + c] = acc;
        }
    }
}

/* ---- fp8 (OCP E4M3) block values with one power-of-two scale per block ----
 * (pytorch_block_sparse summary page and Lecture 11 at 30:31 and 48:12: sparsity combined with
 * quantization; for memory-bound layers the weights are loaded in a compact form and expanded
 * on the GPU before a dense product.)
 *
 * E4M3 as defined by the OCP 8-bit floating point specification: 1 sign bit, 4 exponent bits
 * with bias 7, 3 mantissa bits; exponent field 0 holds the subnormals m * 2^-9; 0x7F and 0xFF
 * are NaN; the largest finite magnitude is 448 = 1.75 * 2^8. */

/* Value of an E4M3 code (NaN codes give NaN). */
double oracle_e4m3_value(uint8_t c)
{
    const int s = c >> 7, E = (c >> 3) & 15, m = c & 7;
    if (E == 15 && m == 7) return NAN;
    const double v = E ? ldexp(1.0 + m / 8.0, E - 7) : ldexp((double)m, -9);
    return s ? -v : v;
}

/* Nearest E4M3 code of x, ties to the even code, |x| <= 448 (the caller guarantees it); the
 * sign of x (also of a zero result) is kept. */
uint8_t oracle_e4m3_encode(double x)
{
    const uint8_t s = signbit(x) ? 0x80 : 0x00;
    const double a = fabs(x);
    if (a < ldexp(1.0, -6)) {                      /* subnormal grid, step 2^-9 */
        const double k = nearbyint(ldexp(a, 9));   /* 0 .. 8; RNE in the default mode */
        if (k >= 8.0) return s | 0x08;             /* rounds up to the smallest normal */
        return s | (uint8_t)k;
    }
    int E;
    const double f = frexp(a, &E);                 /* a = f * 2^E, f in [0.5, 1) */
    double m = nearbyint((2.0 * f - 1.0) * 8.0);   /* mantissa of a = (1 + m/8) 2^(E-1) */
    int e = E - 1;
    if (m >= 8.0) {
        m = 0.0;
        e += 1;
    }
    return s | (uint8_t)((e + 7) << 3) | (uint8_t)m;
}

/* Per block i of n values: amax = max |V[i]|; scale exponent se[i] = the smallest integer
 * e >= -126 with amax <= 448 * 2^e (0 for an all-zero block); codes = E4M3 code of V / 2^se[i]
 * for every value. V is [nnzb][n] (fp64 values of bf16 inputs): n = b*b for dense blocks, b*b/2
 * for the kept values of 2:4 blocks. */
void oracle_quantize_fp8(int32_t nnzb, int32_t n, const double *V, uint8_t *codes, int32_t *se)
{
#pragma omp parallel for schedule(static)
    for (int32_t i = 0; i < nnzb; ++i) {
        const double *v = V + (int64_t)i * n;
        double amax = 0.0;
        for (int32_t k = 0; k < n; ++k)
            if (fabs(v[k]) > amax) amax = fabs(v[k]);
        int32_t e = 0;
        if (amax > 0.0) {
            e = -126;
            while (amax > ldexp(448.0, e)) ++e;
        }
        se[i] = e;
        for (int32_t k = 0; k < n; ++k)
            codes[(int64_t)i * n + k] = oracle_e4m3_encode(ldexp(v[k], -e));
    }
}

/* Dequantised values: code value * 2^se[i], as fp64; [nnzb][n]. */
void oracle_dequantize_fp8(int32_t nnzb, int32_t n, const uint8_t *codes, const int32_t *se, double *V)
{
#pragma omp parallel for schedule(static)
    for (int32_t i = 0; i < nnzb; ++i)
        for (int32_t k = 0; k < n; ++k)
            V[(int64_t)i * n + k] = ldexp(oracle_e4m3_value(codes[(int64_t)i * n + k]), se[i]);
}

/* ---- 2:4 sparsity inside each kept block ----
 * (pytorch_block_sparse summary page, "Future Development Roadmap": the 50% sparse pattern within
 * blocks; pytorch/ao sparsity README: 2:4 semi-structured means two of every four elements are
 * zero, pruned by weight norm over 1 x 4 groups with two zeros per group, stored as a half-size
 * compressed dense matrix plus 2-bit indices (Table 4.1).)
 *
 * Groups are 4 consecutive columns q = 4h .. 4h+3 of one row p of a block (the input dimension,
 * which the forward sums over). In each group the two elements of largest magnitude are kept
 * (ties to the lower position); they are stored in ascending position order:
 *   Vc[i][p][2h + t]   the t-th kept value of group h (t = 0, 1),
 *   meta[i][p][h / 4]  16 bits per 4 groups: group h at bits 4 (h % 4): the first kept position
 *                      in the low 2 bits, the second in the next 2.
 * V is [nnzb][b][b], Vc [nnzb][b][b/2], meta [nnzb][b][b/16]; b a multiple of 16. */
void oracle_compress_24(int32_t nnzb, int32_t b, const double *V, double *Vc, uint16_t *meta)
{
#pragma omp parallel for schedule(static)
    for (int32_t i = 0; i < nnzb; ++i) {
        for (int32_t p = 0; p < b; ++p) {
            const double *v = V + ((int64_t)i * b + p) * b;
            double *vc = Vc + ((int64_t)i * b + p) * (b / 2);
            uint16_t *mt = meta + ((int64_t)i * b + p) * (b / 16);
            for (int32_t w = 0; w < b / 16; ++w) mt[w] = 0;
            for (int32_t h = 0; h < b / 4; ++h) {
                const double *g = v + 4 * h;
                /* first: largest magnitude, lowest position among equals */
                int first = 0;
                for (int k = 1; k < 4; ++k)
                    if (fabs(g[k]) > fabs(g[first])) first = k;
                /* second: largest magnitude among the other three, lowest position among equals */
                int second = -1;
                for (int k = 0; k < 4; ++k) {
                    if (k == first) continue;
                    if (second < 0 || fabs(g[k]) > fabs(g[second])) second = k;
                }
                const int lo = first < second ? first : second, hi = first < second ? second : first;
                vc[2 * h] = g[lo];
                vc[2 * h + 1] = g[hi];
                mt[h / 4] |= (uint16_t)((lo | (hi << 2)) << (4 * (h % 4)));
            }
        }
    }
}

/* Dense blocks from the compressed form: zeros except the two kept positions of every group. */
void oracle_decompress_24(int32_t nnzb, int32_t b, const double *Vc, const uint16_t *meta, double *V)
{
#pragma omp parallel for schedule(static)
    for (int32_t i = 0; i < nnzb; ++i) {
        for (int32_t p = 0; p < b; ++p) {
            const double *vc = Vc + ((int64_t)i * b + p) * (b / 2);
            const uint16_t *mt = meta + ((int64_t)i * b + p) * (b / 16);
            double *v = V + ((int64_t)i * b + p) * b;
            for (int32_t q = 0; q < b; ++q) v[q] = 0.0;
            for (int32_t h = 0; h < b / 4; ++h) {
                const int bits = (mt[h / 4] >> (4 * (h % 4))) & 15;
                v[4 * h + (bits & 3)] = vc[2 * h];
                v[4 * h + (bits >> 2)] = vc[2 * h + 1];
            }
        }
    }
}

/* Threads the OpenMP runtime will use for the loops above. */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the number of threads of the loops above (no effect without OpenMP). Only
 * independent outputs are split over threads, so results do not depend on it. */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
