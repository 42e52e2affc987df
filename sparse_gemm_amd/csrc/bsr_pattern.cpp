// bsr_pattern.cpp -- pattern metadata (CSR, transposed CSC + perm) and kernel work lists.
//
// Formats follow the pytorch/ao sparsity README, Table 4.1: BSR keeps dense blocks plus their
// coordinates; CSR / CSC keep an index pointer (where each row / column starts), the indices
// and the data. Blocks are canonical: ascending column inside a row, ascending row inside a
// column. The transposed form is what the input-gradient kernel walks, so it needs no atomics.
#include <algorithm>
#include <numeric>

#include "bsr_internal.hpp"

namespace bsr {

namespace {

// Transposed metadata by a counting sort over block columns. Rows are visited in ascending
// order, so the rows inside each column come out ascending.
void build_csc(bsr_pattern &p) {
    p.col_ptr.assign(p.C + 1, 0);
    for (int32_t i = 0; i < p.nnzb; ++i) p.col_ptr[p.col_idx[i] + 1]++;
    for (int32_t c = 0; c < p.C; ++c) p.col_ptr[c + 1] += p.col_ptr[c];
    std::vector<int32_t> next(p.col_ptr.begin(), p.col_ptr.end() - 1);
    p.row_idx.assign(p.nnzb, 0);
    p.perm.assign(p.nnzb, 0);
    p.blk_row.assign(p.nnzb, 0);
    for (int32_t r = 0; r < p.R; ++r) {
        for (int32_t i = p.row_ptr[r]; i < p.row_ptr[r + 1]; ++i) {
            const int32_t j = next[p.col_idx[i]]++;
            p.row_idx[j] = r;
            p.perm[j] = i;
            p.blk_row[i] = r;
        }
    }
}

// Output blocks with the most kept blocks first (ties: lower index first).
std::vector<int32_t> by_count_desc(const std::vector<int32_t> &ptr) {
    const int32_t n = (int32_t)ptr.size() - 1;
    std::vector<int32_t> ids(n);
    std::iota(ids.begin(), ids.end(), 0);
    std::stable_sort(ids.begin(), ids.end(), [&](int32_t a, int32_t b) {
        return ptr[a + 1] - ptr[a] > ptr[b + 1] - ptr[b];
    });
    return ids;
}

// Group output blocks (block rows of W for the forward, block columns for the input gradient)
// G at a time in order of decreasing kept-block count. Each group's steps are the union of
// the input blocks its members touch, ascending; a slot's entry is the value block that
// multiplies that input block into that member, or -1.
//   ptr / idx / val: for output block o, entries e in [ptr[o], ptr[o+1]) have input block
//   idx[e] (ascending) and value block val(e).
template <class ValFn>
GroupSchedule make_groups(const std::vector<int32_t> &ptr, const std::vector<int32_t> &idx, ValFn val,
                          int G) {
    GroupSchedule s;
    s.G = G;
    const int32_t nout = (int32_t)ptr.size() - 1;
    const std::vector<int32_t> ids = by_count_desc(ptr);
    s.ngroups = (nout + G - 1) / G;
    s.step_ptr.assign(s.ngroups + 1, 0);
    s.out.assign((size_t)s.ngroups * G, -1);
    std::vector<int32_t> cursor(G);
    for (int32_t g = 0; g < s.ngroups; ++g) {
        int members = 0;
        for (int t = 0; t < G; ++t) {
            const int32_t k = g * G + t;
            if (k < nout) {
                s.out[(size_t)g * G + t] = ids[k];
                cursor[t] = ptr[ids[k]];
                members++;
            }
        }
        // merge the members' ascending input lists
        for (;;) {
            int32_t next_in = INT32_MAX;
            for (int t = 0; t < members; ++t) {
                const int32_t o = s.out[(size_t)g * G + t];
                if (cursor[t] < ptr[o + 1]) next_in = std::min(next_in, idx[cursor[t]]);
            }
            if (next_in == INT32_MAX) break;
            s.step_in.push_back(next_in);
            for (int t = 0; t < G; ++t) {
                int32_t v = -1;
                if (t < members) {
                    const int32_t o = s.out[(size_t)g * G + t];
                    if (cursor[t] < ptr[o + 1] && idx[cursor[t]] == next_in) {
                        v = val(cursor[t]);
                        cursor[t]++;
                    }
                }
                s.step_blk.push_back(v);
            }
        }
        s.step_ptr[g + 1] = (int32_t)s.step_in.size();
    }
    s.order.resize(s.ngroups);
    std::iota(s.order.begin(), s.order.end(), 0);
    std::stable_sort(s.order.begin(), s.order.end(), [&](int32_t a, int32_t b) {
        return s.step_ptr[a + 1] - s.step_ptr[a] > s.step_ptr[b + 1] - s.step_ptr[b];
    });
    return s;
}

}  // namespace

void build_pattern(bsr_pattern &p) {
    build_csc(p);
    const int G = group_size(p.b);
    p.fwd = make_groups(p.row_ptr, p.col_idx, [](int32_t e) { return e; }, G);
    p.bwd = make_groups(p.col_ptr, p.row_idx, [&](int32_t e) { return p.perm[e]; }, G);
    p.rows_by_nnz = by_count_desc(p.row_ptr);
}

}  // namespace bsr
