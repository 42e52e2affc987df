/*
 * bsr_sparse24.h -- 2:4 sparsity inside each kept block (C ABI, same library and conventions as
 * bsr_linear.h: raw bf16 bits, caller-owned contiguous device buffers aligned to 16 bytes, a
 * hipStream_t passed as void*, arguments checked before anything is enqueued, a bsr_status
 * returned, no C++ exception across the interface).
 *
 * The block-sparse layer's roadmap adds the 50% sparse pattern inside blocks (pytorch_block_sparse
 * summary page, "Future Development Roadmap"). 2:4 semi-structured sparsity keeps two of every
 * four consecutive elements; the pytorch/ao sparsity README prunes it by weight norm over 1 x 4
 * groups with two zeros per group (workflow example) and stores it as a half-size compressed
 * matrix plus 2-bit indices (Table 4.1). Here the groups run along a block row's columns (the
 * layer's input dimension, which the forward sums over), so the gfx950 sparse matrix cores can
 * take the compressed block directly.
 *
 * Format of kept block i (CSR order, like V); b = 32 or 64:
 *   Vc[i][p][2h + t]   bf16    the t-th kept value (ascending position) of group h = columns
 *                              4h .. 4h + 3 of row p; [nnzb][b][b/2]
 *   meta[i][p][h / 4]  uint16  group h at bits 4 (h % 4): the first kept position (0..3) in the
 *                              low 2 bits, the second in the next 2; [nnzb][b][b/16]
 * Compression keeps the two elements of largest magnitude of every group, ties to the lower
 * position (for a block that already has at most two nonzeros per group it is lossless).
 */
#ifndef BSR_SPARSE24_H
#define BSR_SPARSE24_H

#include <stddef.h>
#include <stdint.h>

#include "bsr_linear.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Prune bf16 block values V [nnzb][b][b] (device, finite) to 2:4 inside every block row and
 * compress: Vc [nnzb][b][b/2] bf16 and meta [nnzb][b][b/16] uint16 (device). Bit-exact
 * (integer magnitude comparisons). Outputs must not overlap V. */
int32_t bsr_values_compress_24(const bsr_pattern *p, const bsr_bf16 *V, bsr_bf16 *Vc, uint16_t *meta,
                               void *stream);

/* Dense blocks V [nnzb][b][b] from the compressed form: the kept values at their positions, +0.0
 * elsewhere. */
int32_t bsr_values_decompress_24(const bsr_pattern *p, const bsr_bf16 *Vc, const uint16_t *meta,
                                 bsr_bf16 *V, void *stream);

/* Forward with 2:4 block values on the sparse matrix cores: Y[M][N] = X[M][K] . W24~^T + bias,
 * W24~ being the zero-filled weight of the decompressed blocks (the contract of bsr_linear_fwd;
 * bf16 inputs and outputs, fp32 accumulation, one rounding per output). b = 32 with 256 rows or
 * more over block rows kept in most 64-column panels (the condition under which bsr_linear_fwd
 * takes its wide tile) runs that tile on the compressed blocks as they are (1 KB of kept values
 * plus 128 bytes of indices per block, one v_smfmac_f32_32x32x32_bf16 per block and 32 rows; the
 * same accumulation order as bsr_linear_fwd_24_image, so the same result bit for bit). Every other
 * call runs the kernel for few rows (16 rows per pass). Every element of Y is written. Limits: M
 * below 2^20 (BSR_ERR_INVALID_ARG otherwise), the compressed values below 4 GiB; Y must not overlap
 * the inputs. */
int32_t bsr_linear_fwd_24(const bsr_pattern *p, const bsr_bf16 *X, int64_t M, const bsr_bf16 *Vc,
                          const uint16_t *meta, const bsr_bf16 *bias, bsr_bf16 *Y, void *stream);

/* Pack the compressed form into 2:4 block images for the large-M forward: img [nnzb][b][b]
 * (16-bit units, the size of the bf16 blocks): row p of block i holds Vc[i][p][0 .. b/2) (b
 * bytes), then meta[i][p][0 .. b/16) (b/8 bytes), then zeros. */
int32_t bsr_values_pack_24(const bsr_pattern *p, const bsr_bf16 *Vc, const uint16_t *meta, uint16_t *img,
                           void *stream);

/* Forward with 2:4 block images on the sparse matrix cores inside the panel GEMM of
 * bsr_linear_fwd (same work lists, staging and epilogue; one v_smfmac_f32_32x32x32_bf16 per 32
 * columns of a block in place of two dense products): Y[M][N] = X . W24~^T + bias, the contract of
 * bsr_linear_fwd_24, for any M >= 0 (the same limits as bsr_linear_fwd). Y must not overlap the
 * inputs. */
int32_t bsr_linear_fwd_24_image(const bsr_pattern *p, const bsr_bf16 *X, int64_t M, const uint16_t *img,
                                const bsr_bf16 *bias, bsr_bf16 *Y, void *stream);

/* ---- 2:4 combined with fp8 (Lecture 11 summary, 30:31: combining sparsity with quantization) ----
 * The kept values of the compressed form stored as E4M3 codes with one power-of-two scale per
 * block, exactly as in bsr_fp8.h (codes Vc8 [nnzb][b][b/2] uint8, scale exponents se [nnzb] int32,
 * the scale taken over the block's kept values, whose largest magnitude is the block's); the
 * indices stay in meta. */

/* Quantise the kept values Vc [nnzb][b][b/2] (device, finite) into codes Vc8 and exponents se
 * (device, se 4-byte aligned). Bit-exact. */
int32_t bsr_values_quantize_fp8_24(const bsr_pattern *p, const bsr_bf16 *Vc, uint8_t *Vc8, int32_t *se,
                                   void *stream);

/* Forward for few rows with 2:4 blocks of fp8 kept values: the contract of bsr_linear_fwd_24 with
 * the kept values code * 2^se[i] (same limits). */
int32_t bsr_linear_fwd_fp8_24(const bsr_pattern *p, const bsr_bf16 *X, int64_t M, const uint8_t *Vc8,
                              const int32_t *se, const uint16_t *meta, const bsr_bf16 *bias, bsr_bf16 *Y,
                              void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BSR_SPARSE24_H */
