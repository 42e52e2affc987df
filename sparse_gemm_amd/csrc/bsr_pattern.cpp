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
    for (int32_t r = 0; r < p.R; ++r) {
        for (int32_t i = p.row_ptr[r]; i < p.row_ptr[r + 1]; ++i) {
            const int32_t j = next[p.col_idx[i]]++;
            p.row_idx[j] = r;
            p.perm[j] = i;
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
// G at a time in order of decreasing kept-block count. Each group's steps are the union of the
// input blocks its members touch, ascending; a member's value block at a step is the block that
// multiplies that input block into that member, or -1. The steps are then padded and encoded as
// the per-step records described with GroupSchedule.
//   ptr / idx / val: for output block o, entries e in [ptr[o], ptr[o+1]) have input block
//   idx[e] (ascending) and value block val(e).
template <class ValFn>
GroupSchedule make_groups(const std::vector<int32_t> &ptr, const std::vector<int32_t> &idx, ValFn val,
                          int G, int P) {
    GroupSchedule s;
    s.G = G;
    s.P = P;
    s.RS = rec_stride(G);
    s.HS = hdr_stride(G, P);
    const int RS = s.RS, HS = s.HS;
    const int32_t nout = (int32_t)ptr.size() - 1;
    const std::vector<int32_t> ids = by_count_desc(ptr);
    s.ngroups = (nout + G - 1) / G;
    s.step_ptr.assign(s.ngroups + 1, 0);
    s.out.assign((size_t)s.ngroups * G, -1);
    s.hdr.assign((size_t)s.ngroups * HS, -1);
    std::vector<int32_t> cursor(G), in_of, blk_of;   // real steps of the current group
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
        in_of.clear();
        blk_of.clear();
        // merge the members' ascending input lists
        for (;;) {
            int32_t next_in = INT32_MAX;
            for (int t = 0; t < members; ++t) {
                const int32_t o = s.out[(size_t)g * G + t];
                if (cursor[t] < ptr[o + 1]) next_in = std::min(next_in, idx[cursor[t]]);
            }
            if (next_in == INT32_MAX) break;
            in_of.push_back(next_in);
            for (int t = 0; t < G; ++t) {
                int32_t v = -1;
                if (t < members) {
                    const int32_t o = s.out[(size_t)g * G + t];
                    if (cursor[t] < ptr[o + 1] && idx[cursor[t]] == next_in) {
                        v = val(cursor[t]);
                        cursor[t]++;
                    }
                }
                blk_of.push_back(v);
            }
        }
        const int32_t n = (int32_t)in_of.size();
        const int32_t npad = (n + P - 1) / P * P;
        auto in_at = [&](int32_t k) { return n == 0 ? 0 : in_of[std::min(k, n - 1)]; };
        auto blk_at = [&](int32_t k, int t) { return k < n ? blk_of[(size_t)k * G + t] : -1; };
        int32_t *h = &s.hdr[(size_t)g * HS];
        for (int u = 0; u < P; ++u) {
            h[u] = in_at(u);
            for (int t = 0; t < G; ++t) h[P + u * G + t] = blk_at(u, t);
        }
        for (int32_t k = 0; k < npad; ++k) {
            std::vector<int32_t> r(RS, -1);
            int32_t mask = 0;
            for (int t = 0; t < G; ++t)
                if (blk_at(k, t) >= 0) mask |= 1 << t;
            r[0] = mask;
            r[1] = in_at(k + P);
            for (int t = 0; t < G; ++t) r[2 + t] = blk_at(k + P, t);
            s.rec.insert(s.rec.end(), r.begin(), r.end());
        }
        s.step_ptr[g + 1] = s.step_ptr[g] + npad;
    }
    s.order.resize(s.ngroups);
    std::iota(s.order.begin(), s.order.end(), 0);
    std::stable_sort(s.order.begin(), s.order.end(), [&](int32_t a, int32_t b) {
        return s.step_ptr[a + 1] - s.step_ptr[a] > s.step_ptr[b + 1] - s.step_ptr[b];
    });
    return s;
}

// Weight-gradient runs: every block row is cut into runs of at most GB consecutive kept
// blocks; runs with more blocks come first.
DwSchedule make_dw_groups(const bsr_pattern &p, int GB) {
    DwSchedule s;
    s.GB = GB;
    std::vector<int32_t> row, first, count;
    for (int32_t r = 0; r < p.R; ++r) {
        for (int32_t i = p.row_ptr[r]; i < p.row_ptr[r + 1]; i += GB) {
            row.push_back(r);
            first.push_back(i);
            count.push_back(std::min<int32_t>(GB, p.row_ptr[r + 1] - i));
        }
    }
    s.ngroups = (int)row.size();
    std::vector<int32_t> ids(s.ngroups);
    std::iota(ids.begin(), ids.end(), 0);
    std::stable_sort(ids.begin(), ids.end(), [&](int32_t a, int32_t b) { return count[a] > count[b]; });
    for (int32_t k : ids) {
        s.row.push_back(row[k]);
        s.first.push_back(first[k]);
        s.count.push_back(count[k]);
    }
    return s;
}

}  // namespace

void build_pattern(bsr_pattern &p) {
    build_csc(p);
    const int Gs[2] = {wide_group(p.b), narrow_group(p.b)};
    for (int k = 0; k < 2; ++k) {
        p.fwd[k] = make_groups(p.row_ptr, p.col_idx, [](int32_t e) { return e; }, Gs[k], gemm_depth(p.b));
        p.bwd[k] = make_groups(p.col_ptr, p.row_idx, [&](int32_t e) { return p.perm[e]; }, Gs[k], gemm_depth(p.b));
    }
    p.dw = make_dw_groups(p, dw_group(p.b));
    p.rows_by_nnz = by_count_desc(p.row_ptr);
}

}  // namespace bsr
