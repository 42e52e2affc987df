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

#ifdef __cplusplus
}
#endif

#endif /* BSR_REBUILD_H */
