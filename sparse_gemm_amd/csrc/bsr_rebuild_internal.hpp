// bsr_rebuild_internal.hpp -- launcher of the on-device metadata rebuild (include/bsr_rebuild.h).
#pragma once

#include <cstddef>
#include <cstdint>

#include "bsr_internal.hpp"
#include "bsr_rebuild.h"

namespace bsr {

size_t rebuild_workspace_bytes(int32_t R, int32_t C);
// capped: the CSC lists keep only the blocks whose CSR position lies below cap (device-built
// patterns); otherwise they are bsr_meta_rebuild's (CSC positions at or past cap not written).
int32_t launch_rebuild(int32_t R, int32_t C, const uint8_t *mask, int32_t *row_ptr, int32_t *col_idx,
                       int32_t *col_ptr, int32_t *row_idx, int32_t *perm, int32_t cap, int32_t *nnzb, void *ws,
                       void *stream, bool capped = false);

// Device-built patterns (bsr_pattern_create_device): scratch bytes of the work-list builders, and
// the rebuild of metadata and work lists from a device mask.
size_t sched_scratch_bytes(int32_t R, int32_t C, int b);
int32_t launch_pattern_rebuild(const bsr_pattern &p, const uint8_t *mask, void *stream);

// bsr_kernels.hip: the small-M forward reading a device CSR row pointer in natural row order.
int32_t launch_small_m_fwd_csr(int32_t N, int32_t K, int32_t b, const int32_t *row_ptr, const int32_t *col_idx,
                               int32_t cap, const FwdArgs &a, void *stream);

}  // namespace bsr
