/*
 * bsr_rebuild.h -- the pattern metadata rebuilt on the device from a block mask (C ABI, same
 * library and conventions as bsr_linear.h; a hipStream_t passed as void*; arguments checked before
 * anything is enqueued; a bsr_status returned; no C++ exception across the interface).
 *
 * The roadmap moves beyond patterns fixed at initialisation (pytorch_block_sparse summary page,
 * "Future Development Roadmap"); out-of-place mask updates let pruned weights grow back when the
 * mask changes (pytorch/ao sparsity README, criteria list). This call rebuilds the index arrays of
 * a changed mask where the mask lives, asynchronously and with no host synchronisation (usable
 * inside a training loop or a captured graph): the CSR index pointer and block columns, and the
 * transposed CSC form with perm, defined exactly as in bsr_linear.h (canonical ascending orders),
 * so the result equals bsr_pattern_export of a pattern built from the same mask, bit for bit.
 * bsr_meta_rebuild writes the arrays to caller buffers. A device-built pattern
 * (bsr_pattern_create_device, bsr_pattern_rebuild) goes further: it rebuilds the metadata and the
 * compute kernels' work lists in place from a changed mask, so the forward, the input gradient and
 * the weight gradient follow the new mask with no host round trip, inside a captured graph too.
 */
#ifndef BSR_REBUILD_H
#define BSR_REBUILD_H

#include <stddef.h>
#include <stdint.h>

#include "bsr_linear.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of device workspace bsr_meta_rebuild needs for an R x C block grid. */
size_t bsr_meta_rebuild_workspace(int32_t R, int32_t C);

/* Rebuild the metadata of the device block mask [R][C] (uint8, row-major, nonzero = kept):
 *   row_ptr[R+1], col_ptr[C+1]           int32 device outputs, always written in full;
 *   col_idx, row_idx, perm [cap]         int32 device outputs; entries at positions >= cap are
 *                                        not written (pass cap = R*C to always get all of them);
 *   nnzb                                 int32 device output: the number of kept blocks (which
 *                                        may exceed cap: then the index arrays are incomplete);
 *   workspace / ws_bytes                 caller-owned device scratch of at least
 *                                        bsr_meta_rebuild_workspace(R, C) bytes.
 * R, C > 0 with R < 2^31 / C; device pointers must be 4-byte aligned; outputs must not overlap
 * each other, the mask or the workspace. Deterministic (integer scans, no atomics). */
int32_t bsr_meta_rebuild(int32_t R, int32_t C, const uint8_t *mask, int32_t *row_ptr, int32_t *col_idx,
                         int32_t *col_ptr, int32_t *row_idx, int32_t *perm, int32_t cap, int32_t *nnzb,
                         void *workspace, size_t ws_bytes, void *stream);

/* Forward for few activation rows straight from device CSR metadata (for example the output of
 * bsr_meta_rebuild), with no pattern object and no host round trip: Y[M][N] = X[M][K] . W~^T + bias
 * where block row r keeps the blocks row_ptr[r] .. row_ptr[r+1]-1 with columns col_idx[...] and
 * values V[...] in that order (the contract of bsr_linear_fwd). The work-groups take the block rows
 * in natural order (the host-built pattern deals them heaviest first).
 *   N, K, b   as for a pattern (b = 32 or 64, N and K positive multiples of b).
 *   row_ptr   device int32 [N/b + 1]: canonical CSR (non-decreasing, starting at 0).
 *   col_idx   device int32 [cap]: block columns, ascending and in range inside each row.
 *   cap       the number of blocks col_idx and V hold (>= 0). Block positions at or past cap are
 *             dropped: a row keeps only its blocks below cap. This is the truncation
 *             bsr_meta_rebuild applies when a mask holds more than its capacity (its row_ptr is
 *             written in full, its col_idx only below cap), so a grown mask never makes this call
 *             read past col_idx or V. Pass bsr_meta_rebuild's cap; compare its nnzb output with
 *             cap to detect the truncation.
 *   The metadata is not validated on the host, since it lives on the device: malformed
 *   metadata is the caller's error, but loads stay inside X, V (cap blocks) and col_idx.
 *   X [M][K], V [cap][b][b], bias [N] or NULL, Y [M][N]: bf16 device buffers, 16-byte aligned;
 *             1 <= M <= 16 (M = 0 is a no-op); cap * b * b values below 4 GiB.
 * Every element of Y is written. */
int32_t bsr_linear_fwd_small_m_csr(int32_t N, int32_t K, int32_t b, const int32_t *row_ptr,
                                   const int32_t *col_idx, int32_t cap, const bsr_bf16 *X, int64_t M,
                                   const bsr_bf16 *V, const bsr_bf16 *bias, bsr_bf16 *Y, void *stream);

/* A pattern whose metadata and work lists live on the device only, for masks that change during
 * training (pytorch_block_sparse summary page, "Future Development Roadmap": beyond patterns fixed
 * at initialisation; pytorch/ao sparsity README, criteria list: out-of-place mask updates let
 * weights regrow). Created once per layer, outside any captured graph (it allocates), with a
 * capacity: the most kept blocks any mask it will take may hold.
 *   N, K, b  as for bsr_pattern_create_from_mask.
 *   cap      1 <= cap <= min(2^23 - 1, (N/b)*(K/b)).
 * The new pattern is empty (no kept block) until bsr_pattern_rebuild. It serves bsr_linear_fwd,
 * bsr_linear_bwd_input, bsr_linear_bwd_weight(_noalloc), bsr_linear_bwd_weight_workspace,
 * bsr_op_kernels, bsr_pattern_info (which reports nnzb = cap) and bsr_pattern_destroy; other
 * calls return BSR_ERR_UNSUPPORTED. For it, V and dV hold cap blocks ([cap][b][b]): the blocks of
 * the current mask in CSR order first; dV positions at or past the live count are unspecified.
 * The compute calls size their grids by the capacity and read the live work lists on the device
 * (the forward takes 16 rows or fewer on the streaming kernel, natural row order; more rows on the
 * panel GEMM's 4-member groups in natural order; the weight gradient on its tile items). Each
 * output equals, bit for bit, what a host-built pattern of the same mask gives when both run the
 * same kernel configuration. Released with bsr_pattern_destroy. */
int32_t bsr_pattern_create_device(int32_t N, int32_t K, int32_t b, int32_t cap, bsr_pattern **out);

/* Rebuild a device-built pattern from the device block mask [N/b][K/b] (uint8, row-major,
 * nonzero = kept) on `stream`, with no host synchronisation (capturable): the metadata exactly as
 * bsr_meta_rebuild with the pattern's capacity (a mask holding more than cap blocks keeps, in
 * every list, only the blocks whose CSR position lies below cap), then the forward's and the input
 * gradient's group work lists and the weight gradient's items from it. Compute calls enqueued after
 * it on the same stream see the new mask. BSR_ERR_UNSUPPORTED for a host-built pattern. */
int32_t bsr_pattern_rebuild(bsr_pattern *p, const uint8_t *mask, void *stream);

/* Device pointers of a device-built pattern's metadata (valid until bsr_pattern_destroy, contents
 * as of the last completed rebuild): row_ptr [N/b+1], col_idx [cap], col_ptr [K/b+1], row_idx
 * [cap], perm [cap] (the arrays of bsr_meta_rebuild) and nnzb [1], the live number of kept blocks
 * (which may exceed cap). Any output may be NULL. Host only, no device access. */
int32_t bsr_pattern_device_arrays(const bsr_pattern *p, const int32_t **row_ptr, const int32_t **col_idx,
                                  const int32_t **col_ptr, const int32_t **row_idx, const int32_t **perm,
                                  const int32_t **nnzb);

#ifdef __cplusplus
}
#endif

#endif /* BSR_REBUILD_H */
