// bsr_select.cpp -- host half of the block-magnitude pattern selection.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "bsr_convert_internal.hpp"

namespace bsr {

// The `keep` blocks with the largest norm (pytorch/ao sparsity README, Table 4.2: the magnitude
// criterion removes the lowest norms), ties going to the lower row-major index r * C + c. Ordering
// by (norm descending, index ascending) is a total order, so the mask is unique; nth_element puts
// exactly the first `keep` blocks of that order in front.
int32_t mask_topk(int32_t R, int32_t C, const double *norms, int64_t keep, uint8_t *mask) {
    const int64_t n = (int64_t)R * C;
    std::vector<int64_t> idx((size_t)n);
    for (int64_t i = 0; i < n; ++i) {
        if (std::isnan(norms[i])) return fail(BSR_ERR_INVALID_ARG, "a block norm is NaN");
        idx[(size_t)i] = i;
    }
    std::memset(mask, 0, (size_t)n);
    if (keep >= n) {
        std::memset(mask, 1, (size_t)n);
        return BSR_OK;
    }
    auto before = [norms](int64_t a, int64_t b) { return norms[a] > norms[b] || (norms[a] == norms[b] && a < b); };
    if (keep > 0) std::nth_element(idx.begin(), idx.begin() + (keep - 1), idx.end(), before);
    for (int64_t k = 0; k < keep; ++k) mask[idx[(size_t)k]] = 1;
    return BSR_OK;
}

}  // namespace bsr
