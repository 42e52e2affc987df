/* The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only, built with gcc by
 * tests/test_sanitizers.py): every entry point runs on small seeded inputs whose shapes include
 * empty rows and columns, single blocks and both block sizes; the forward, input gradient and
 * weight gradient are compared with the dense product of the zero-filled weight (exact here:
 * small-integer inputs make every sum exact in fp64). Prints "OK" and exits 0 when all hold. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void oracle_fwd(int64_t M, int32_t N, int32_t K, int32_t b, const int32_t *row_ptr, const int32_t *col_idx,
                const double *X, const double *V, const double *bias, double *Y, double *S);
void oracle_dx(int64_t M, int32_t N, int32_t K, int32_t b, const int32_t *row_ptr, const int32_t *col_idx,
               const double *dY, const double *V, double *dX, double *S);
void oracle_dw(int64_t M, int32_t N, int32_t K, int32_t b, const int32_t *row_ptr, const int32_t *col_idx,
               const double *dY, const double *X, const int32_t *blocks, int32_t nblocks, double *dV, double *S);
void oracle_db(int64_t M, int32_t N, const double *dY, double *db, double *S);
void oracle_block_norms(int32_t N, int32_t K, int32_t b, int32_t kind, const double *W, double *norms);
double oracle_e4m3_value(uint8_t c);
uint8_t oracle_e4m3_encode(double x);
void oracle_quantize_fp8(int32_t nnzb, int32_t n, const double *V, uint8_t *codes, int32_t *se);
void oracle_dequantize_fp8(int32_t nnzb, int32_t n, const uint8_t *codes, const int32_t *se, double *V);
void oracle_compress_24(int32_t nnzb, int32_t b, const double *V, double *Vc, uint16_t *meta);
void oracle_decompress_24(int32_t nnzb, int32_t b, const double *Vc, const uint16_t *meta, double *V);

static int fails = 0;
#define REQUIRE(c)                                                              \
    do {                                                                        \
        if (!(c)) {                                                             \
            fprintf(stderr, "%s:%d: %s failed\n", __FILE__, __LINE__, #c);      \
            if (++fails > 20) exit(1);                                          \
        }                                                                       \
    } while (0)

static uint64_t st = 88172645463325252ull;
static uint32_t rnd(void) {
    st ^= st << 13;
    st ^= st >> 7;
    st ^= st << 17;
    return (uint32_t)(st >> 16);
}
static double small_int(void) { return (double)((int)(rnd() % 5) - 2); }

static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) exit(2);
    return p;
}

static void run_case(int64_t M, int32_t R, int32_t C, int32_t b, int density_pct) {
    const int32_t N = R * b, K = C * b;
    uint8_t *mask = xmalloc((size_t)R * C);
    int32_t *row_ptr = xmalloc(sizeof(int32_t) * (size_t)(R + 1));
    int32_t *col_idx = xmalloc(sizeof(int32_t) * (size_t)R * C);
    int32_t n = 0;
    row_ptr[0] = 0;
    for (int32_t r = 0; r < R; ++r) {
        for (int32_t c = 0; c < C; ++c) {
            mask[(size_t)r * C + c] = (int)(rnd() % 100) < density_pct;
            if (mask[(size_t)r * C + c]) col_idx[n++] = c;
        }
        row_ptr[r + 1] = n;
    }
    double *X = xmalloc(sizeof(double) * (size_t)(M * K)), *dY = xmalloc(sizeof(double) * (size_t)(M * N));
    double *V = xmalloc(sizeof(double) * (size_t)n * b * b), *bias = xmalloc(sizeof(double) * (size_t)N);
    double *W = xmalloc(sizeof(double) * (size_t)N * K);
    for (int64_t i = 0; i < M * K; ++i) X[i] = small_int();
    for (int64_t i = 0; i < M * N; ++i) dY[i] = small_int();
    for (int64_t i = 0; i < (int64_t)n * b * b; ++i) V[i] = small_int();
    for (int32_t i = 0; i < N; ++i) bias[i] = small_int();
    memset(W, 0, sizeof(double) * (size_t)N * K);
    for (int32_t r = 0; r < R; ++r)
        for (int32_t i = row_ptr[r]; i < row_ptr[r + 1]; ++i)
            for (int32_t p = 0; p < b; ++p)
                for (int32_t q = 0; q < b; ++q) W[(size_t)(r * b + p) * K + col_idx[i] * b + q] = V[((size_t)i * b + p) * b + q];
    double *Y = xmalloc(sizeof(double) * (size_t)(M * N)), *S = xmalloc(sizeof(double) * (size_t)(M * (N > K ? N : K)));
    oracle_fwd(M, N, K, b, row_ptr, col_idx, X, V, bias, Y, S);
    for (int64_t m = 0; m < M; ++m)
        for (int32_t j = 0; j < N; ++j) {
            double acc = bias[j];
            for (int32_t k = 0; k < K; ++k) acc += X[m * K + k] * W[(size_t)j * K + k];
            REQUIRE(Y[m * N + j] == acc);
        }
    double *dX = xmalloc(sizeof(double) * (size_t)(M * K));
    oracle_dx(M, N, K, b, row_ptr, col_idx, dY, V, dX, S);
    for (int64_t m = 0; m < M; ++m)
        for (int32_t k = 0; k < K; ++k) {
            double acc = 0;
            for (int32_t j = 0; j < N; ++j) acc += dY[m * N + j] * W[(size_t)j * K + k];
            REQUIRE(dX[m * K + k] == acc);
        }
    double *dV = xmalloc(sizeof(double) * (size_t)n * b * b), *SV = xmalloc(sizeof(double) * (size_t)n * b * b);
    oracle_dw(M, N, K, b, row_ptr, col_idx, dY, X, NULL, n, dV, SV);
    for (int32_t r = 0; r < R; ++r)
        for (int32_t i = row_ptr[r]; i < row_ptr[r + 1]; ++i)
            for (int32_t p = 0; p < b; ++p)
                for (int32_t q = 0; q < b; ++q) {
                    double acc = 0;
                    for (int64_t m = 0; m < M; ++m) acc += dY[m * N + r * b + p] * X[m * K + col_idx[i] * b + q];
                    REQUIRE(dV[((size_t)i * b + p) * b + q] == acc);
                }
    if (n > 1) {   /* a block subset, in reverse order */
        int32_t blocks[2] = {n - 1, 0};
        oracle_dw(M, N, K, b, row_ptr, col_idx, dY, X, blocks, 2, dV, NULL);
    }
    double *db = xmalloc(sizeof(double) * (size_t)N), *Sb = xmalloc(sizeof(double) * (size_t)N);
    oracle_db(M, N, dY, db, Sb);
    double *norms = xmalloc(sizeof(double) * (size_t)R * C);
    oracle_block_norms(N, K, b, 1, W, norms);
    oracle_block_norms(N, K, b, 2, W, norms);
    uint8_t *codes = xmalloc((size_t)n * b * b);
    int32_t *se = xmalloc(sizeof(int32_t) * (size_t)(n ? n : 1));
    oracle_quantize_fp8(n, b * b, V, codes, se);
    oracle_dequantize_fp8(n, b * b, codes, se, dV);
    double *Vc = xmalloc(sizeof(double) * (size_t)n * b * b / 2);
    uint16_t *meta = xmalloc(sizeof(uint16_t) * (size_t)n * b * b / 16);
    oracle_compress_24(n, b, V, Vc, meta);
    oracle_decompress_24(n, b, Vc, meta, dV);
    free(mask); free(row_ptr); free(col_idx); free(X); free(dY); free(V); free(bias); free(W); free(Y); free(S);
    free(dX); free(dV); free(SV); free(db); free(Sb); free(norms); free(codes); free(se); free(Vc); free(meta);
}

int main(void) {
    run_case(3, 2, 3, 4, 50);
    run_case(1, 1, 1, 2, 100);
    run_case(5, 3, 2, 4, 0);
    run_case(4, 4, 4, 8, 30);
    run_case(2, 2, 2, 32, 60);
    run_case(0, 2, 2, 4, 50);
    for (int c = 0; c < 256; ++c) {
        const double v = oracle_e4m3_value((uint8_t)c);
        if (!isnan(v)) REQUIRE(oracle_e4m3_value(oracle_e4m3_encode(v)) == v);
    }
    if (fails) {
        fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    printf("OK\n");
    return 0;
}
