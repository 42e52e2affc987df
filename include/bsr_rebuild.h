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
 * The kernels' work lists are host-built: a pattern for the compute calls is still created with
 * bsr_pattern_create_from_csr from these arrays once they are on the host.
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

#ifdef __cplusplus
}
#endif

#endif /* BSR_REBUILD_H */
