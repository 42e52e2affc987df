// bsr_convert_internal.hpp -- launchers and host helpers of the dense <-> BSR conversion and the
// block-magnitude selection (include/bsr_convert.h). All return a bsr_status.
#pragma once

#include <cstdint>

#include "bsr_convert.h"
#include "bsr_internal.hpp"

namespace bsr {

// bsr_convert.hip
int32_t launch_block_norms(int32_t N, int32_t K, int32_t b, const uint16_t *W, int32_t kind, double *norms,
                           void *stream);
int32_t launch_dense_to_values(const bsr_pattern &p, const uint16_t *W, uint16_t *V, void *stream);
int32_t launch_values_to_dense(const bsr_pattern &p, const uint16_t *V, uint16_t *W, void *stream);

// bsr_select.cpp: the `keep` largest block norms, ties to the lower row-major index.
int32_t mask_topk(int32_t R, int32_t C, const double *norms, int64_t keep, uint8_t *mask);

}  // namespace bsr
