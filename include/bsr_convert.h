/*
 * bsr_convert.h -- dense <-> BSR conversion and block-magnitude pattern selection (C ABI,
 * same library and conventions as bsr_linear.h: raw bf16 bits, caller-owned contiguous
 * row-major device buffers aligned to 16 bytes, a hipStream_t passed as void*, arguments
 * checked before anything is enqueued, a bsr_status returned, no C++ exception across the
 * interface).
 *
 * The hand-off between a pruning front end and the sparse kernels is a dense weight with
 * zeros in the dropped places (pytorch/ao sparsity README, workflow section). BSR keeps the
 * dense blocks plus their coordinates (README Table 4.1). The most common pruning criterion
 * is weight magnitude: the parameters with the lowest norm are removed, L1 being the usual
 * norm (README Table 4.2 and the criteria list, which also names the layer-local scope and
 * scoring from the weight tensor alone). At block granularity this chooses the pattern of a
 * BlockSparseLinear layer (pytorch_block_sparse summary page, "Future Development Roadmap":
 * measuring parameter usefulness to choose the pattern).
 *
 * Pipeline: bsr_block_norms (device) -> bsr_mask_topk (host) -> bsr_pattern_create_from_mask
 * -> bsr_dense_to_values (device); bsr_pattern_create_from_dense runs the first three in one
 * call. bsr_values_to_dense gives the dense hand-off form back.
 */
#ifndef BSR_CONVERT_H
#define BSR_CONVERT_H

#include <stddef.h>
#include <stdint.h>

#include "bsr_linear.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Norms for bsr_block_norms / bsr_pattern_create_from_dense. */
enum bsr_norm_kind {
    BSR_NORM_L1 = 1,        /* sum of |w| over the block */
    BSR_NORM_L2_SQUARED = 2 /* sum of w*w over the block (same order as the L2 norm) */
};

/* Block magnitudes of a dense weight.
 *   N, K   weight shape (out, in), positive multiples of b; b = 32 or 64
 *          (BSR_ERR_UNSUPPORTED otherwise); N/b below 65536.
 *   W      device [N][K] bf16.
 *   kind   BSR_NORM_L1 or BSR_NORM_L2_SQUARED.
 *   norms  device [N/b][K/b] fp64 output, row-major over the block grid:
 *          norms[r][c] = sum over p ascending of (sum over q ascending of t(W[r*b+p][c*b+q])),
 *          t = |w| or w*w, each sum left to right in fp64 from 0. Every term is exact in fp64
 *          and the order is fixed, so the result is reproducible bit for bit (and the same
 *          on any launch shape). Must not overlap W.
 * Asynchronous on `stream`. */
int32_t bsr_block_norms(int32_t N, int32_t K, int32_t b, const bsr_bf16 *W, int32_t kind, double *norms,
                        void *stream);

/* Host: mask of the `keep` blocks with the largest norm, ties to the lower row-major index
 * r*C + c (so the mask is unique).
 *   norms  host [R][C] fp64 (a NaN gives BSR_ERR_INVALID_ARG; +Inf ranks highest).
 *   keep   0 .. R*C.
 *   mask   host [R][C] output, 1 = kept, 0 = dropped. */
int32_t bsr_mask_topk(int32_t R, int32_t C, const double *norms, int64_t keep, uint8_t *mask);

/* Pattern of the `keep` blocks of largest norm of the dense device weight W [N][K]: runs
 * bsr_block_norms on `stream`, waits for it (the call is synchronous, like every pattern
 * creation), then bsr_mask_topk and bsr_pattern_create_from_mask with upload. It allocates
 * and frees a temporary [N/b][K/b] fp64 device buffer. `out` receives the new pattern. */
int32_t bsr_pattern_create_from_dense(int32_t N, int32_t K, int32_t b, const bsr_bf16 *W, int32_t kind,
                                      int64_t keep, void *stream, bsr_pattern **out);

/* Read the kept blocks of a dense weight into BSR order: V[i][p][q] = W[r*b+p][col_idx[i]*b+q]
 * for every kept block i (CSR order). W device [N][K] bf16; V device [nnzb][b][b] bf16 output,
 * must not overlap W. Values are copied bit for bit. */
int32_t bsr_dense_to_values(const bsr_pattern *p, const bsr_bf16 *W, bsr_bf16 *V, void *stream);

/* The dense hand-off form: W~[N][K] with block (r, col_idx[i]) = V[i] and +0.0 elsewhere.
 * V device [nnzb][b][b] bf16; W device [N][K] bf16 output, every element written; must not
 * overlap V. Values are copied bit for bit. N/b must be below 65536. */
int32_t bsr_values_to_dense(const bsr_pattern *p, const bsr_bf16 *V, bsr_bf16 *W, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BSR_CONVERT_H */
