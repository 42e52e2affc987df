/*
 * bsr_fp8.h -- fp8 block values for the block-sparse linear layer (C ABI, same library and
 * conventions as bsr_linear.h: raw bf16 bits, caller-owned contiguous device buffers aligned to
 * 16 bytes, a hipStream_t passed as void*, arguments checked before anything is enqueued, a
 * bsr_status returned, no C++ exception across the interface).
 *
 * Memory-bound layers gain from loading the weights in a compact form and expanding them on the
 * GPU before the dense product (Lecture 11 summary, 48:12 "Load and Sparse Expand"); sparsity
 * combines with quantization (same summary, 30:31; pytorch/ao sparsity README: sparsity composes
 * with the quantization workflows). Here each kept block's values are stored as 8-bit floats with
 * one power-of-two scale per block, halving the bytes of the block values.
 *
 * Format of kept block i (i in CSR order, like V):
 *   V8[i][p][q]  uint8  an E4M3 code as defined by the OCP 8-bit floating point specification
 *                (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
 *                holds the subnormals m * 2^-9; largest finite magnitude 448; 0x7F / 0xFF NaN).
 *   se[i]        int32  scale exponent: the element's value is code * 2^se[i].
 * Quantisation: se[i] is the smallest integer >= -126 with max |V[i]| <= 448 * 2^se[i] (0 for an
 * all-zero block); each code is V[i][p][q] / 2^se[i] rounded to the nearest E4M3 value, ties to
 * the even code, sign kept (so no code is NaN). The relative error of a value in the normal range
 * is at most 2^-4.
 */
#ifndef BSR_FP8_H
#define BSR_FP8_H

#include <stddef.h>
#include <stdint.h>

#include "bsr_linear.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Quantise bf16 block values V [nnzb][b][b] (device, finite values) into codes V8 [nnzb][b][b]
 * (device uint8) and scale exponents se [nnzb] (device int32, 4-byte aligned). Deterministic
 * and bit-exact (integer rounding on exact values). Outputs must not overlap V. */
int32_t bsr_values_quantize_fp8(const bsr_pattern *p, const bsr_bf16 *V, uint8_t *V8, int32_t *se,
                                void *stream);

/* Expand codes back to bf16: V[i][p][q] = code * 2^se[i] (exact when the result is a bf16 value,
 * which holds for every block whose largest magnitude is at least 2^-115). */
int32_t bsr_values_dequantize_fp8(const bsr_pattern *p, const uint8_t *V8, const int32_t *se,
                                  bsr_bf16 *V, void *stream);

/* Forward with fp8 block values: Y[M][N] = X[M][K] . W8~^T + bias, where W8~ is the zero-filled
 * weight whose kept block i holds code * 2^se[i] (the same contract as bsr_linear_fwd with the
 * dequantised values; bf16 inputs and outputs, fp32 accumulation, one rounding per output).
 * Built for few activation rows (decode; 16 rows per pass, any M >= 0 with M below 2^20 and
 * 16 rows of X below 4 GiB). Every element of Y is written; rows of W with no kept block give
 * bias (or 0). Y must not overlap X, V8, se or bias. */
int32_t bsr_linear_fwd_fp8(const bsr_pattern *p, const bsr_bf16 *X, int64_t M, const uint8_t *V8,
                           const int32_t *se, const bsr_bf16 *bias, bsr_bf16 *Y, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BSR_FP8_H */
