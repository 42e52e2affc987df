// bsr_fp8_internal.hpp -- launchers of the fp8 block-value kernels (include/bsr_fp8.h).
#pragma once

#include <cstdint>

#include "bsr_fp8.h"
#include "bsr_internal.hpp"

namespace bsr {

// kept24: V holds the kept values of 2:4 blocks ([nnzb][b][b/2]) instead of dense blocks.
int32_t launch_quantize_fp8(const bsr_pattern &p, const uint16_t *V, uint8_t *V8, int32_t *se, void *stream,
                            bool kept24 = false);
int32_t launch_dequantize_fp8(const bsr_pattern &p, const uint8_t *V8, const int32_t *se, uint16_t *V, void *stream);
int32_t launch_fwd_fp8(const bsr_pattern &p, const uint16_t *X, int64_t M, const uint8_t *V8, const int32_t *se,
                       const uint16_t *bias, uint16_t *Y, void *stream);

}  // namespace bsr
