// bsr_sparse24_internal.hpp -- launchers of the 2:4-inside-blocks kernels (include/bsr_sparse24.h).
#pragma once

#include <cstdint>

#include "bsr_internal.hpp"
#include "bsr_sparse24.h"

namespace bsr {

int32_t launch_compress_24(const bsr_pattern &p, const uint16_t *V, uint16_t *Vc, uint16_t *meta, void *stream);
int32_t launch_decompress_24(const bsr_pattern &p, const uint16_t *Vc, const uint16_t *meta, uint16_t *V,
                             void *stream);
int32_t launch_pack_24(const bsr_pattern &p, const uint16_t *Vc, const uint16_t *meta, uint16_t *img, void *stream);
int32_t launch_fwd_24(const bsr_pattern &p, const uint16_t *X, int64_t M, const uint16_t *Vc, const uint16_t *meta,
                      const uint16_t *bias, uint16_t *Y, void *stream);

int32_t launch_fwd_fp8_24(const bsr_pattern &p, const uint16_t *X, int64_t M, const uint8_t *Vc8, const int32_t *se,
                          const uint16_t *meta, const uint16_t *bias, uint16_t *Y, void *stream);

}  // namespace bsr
