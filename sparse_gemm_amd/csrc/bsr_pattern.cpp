// bsr_pattern.cpp -- pattern metadata (CSR, transposed CSC + perm) and kernel work lists.
//
// Formats follow the pytorch/ao sparsity README, Table 4.1: BSR keeps dense blocks plus their
// coordinates; CSR / CSC keep an index pointer (where each row / column starts), the indices
// and the data. Blocks are canonical: ascending column inside a row, ascending row inside a
// column. The transposed form is what the input-gradient kernel walks, so it needs no atomics.
#include <algorithm>
#include <numeric>
#include <utility>

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
// G at a time in order of decreasing kept-block count, so that a group's members need similar
// numbers of panels. A group's work list is the activation panels (kPanelCols columns, i.e.
// kPanelCols / b input blocks) in which any member has a kept block, ascending; the units of a
// panel (member t, block h inside the panel: unit t * PB + h) that have kept blocks go S at a time
// into sub-steps, in unit order.
//   ptr / idx / val: for output block o, entries e in [ptr[o], ptr[o+1]) have input block
//   idx[e] (ascending) and value block val(e).
template <class ValFn>
GroupSchedule make_panels(const std::vector<int32_t> &ptr, const std::vector<int32_t> &idx, ValFn val, int b, int G,
                          int S) {
    const int PB = kPanelCols / b;
    const int U = G * PB;
    const int32_t nout = (int32_t)ptr.size() - 1;
    const std::vector<int32_t> ids = by_count_desc(ptr);
    GroupSchedule s;
    s.G = G;
    s.S = S;
    s.ngroups = (nout + G - 1) / G;
    s.out.assign((size_t)s.ngroups * G, -1);
    s.sub_ptr.assign(s.ngroups + 1, 0);
    std::vector<int32_t> cursor(G), unit_blk(U);
    for (int32_t g = 0; g < s.ngroups; ++g) {
        int members = 0;
        for (int t = 0; t < G && g * G + t < nout; ++t, ++members) {
            s.out[(size_t)g * G + t] = ids[g * G + t];
            cursor[t] = ptr[ids[g * G + t]];
        }
        int32_t nsub = 0;
        for (;;) {
            int32_t panel = INT32_MAX;
            for (int t = 0; t < members; ++t) {
                const int32_t o = s.out[(size_t)g * G + t];
                if (cursor[t] < ptr[o + 1]) panel = std::min(panel, idx[cursor[t]] / PB);
            }
            if (panel == INT32_MAX) break;
            std::fill(unit_blk.begin(), unit_blk.end(), -1);
            for (int t = 0; t < members; ++t) {
                const int32_t o = s.out[(size_t)g * G + t];
                while (cursor[t] < ptr[o + 1] && idx[cursor[t]] / PB == panel) {
                    unit_blk[t * PB + idx[cursor[t]] % PB] = val(cursor[t]);
                    cursor[t]++;
                }
            }
            int u = 0;
            while (u < U) {
                std::vector<int32_t> r(kRecInts, -1);
                r[0] = panel;
                uint32_t map[2] = {0xffffffffu, 0xffffffffu};
                int k = 0;
                for (; u < U && k < S; ++u) {
                    if (unit_blk[u] < 0) continue;
                    r[1 + k] = unit_blk[u];
                    map[u / 8] &= ~(15u << (4 * (u % 8)));
                    map[u / 8] |= (uint32_t)k << (4 * (u % 8));
                    ++k;
                }
                if (k == 0) break;   // no kept blocks left in this panel
                r[1 + S] = (int32_t)map[0];
                r[2 + S] = (int32_t)map[1];
                s.rec.insert(s.rec.end(), r.begin(), r.end());
                ++nsub;
            }
        }
        s.sub_ptr[g + 1] = s.sub_ptr[g] + nsub;
    }
    s.order.resize(s.ngroups);
    std::iota(s.order.begin(), s.order.end(), 0);
    std::stable_sort(s.order.begin(), s.order.end(), [&](int32_t a, int32_t b) {
        return s.sub_ptr[a + 1] - s.sub_ptr[a] > s.sub_ptr[b + 1] - s.sub_ptr[b];
    });
    return s;
}

// Weight-gradient items. Block rows are taken in groups of TR, most kept blocks first. Inside a
// group, a column holding kept blocks in at least half of the group's rows costs one shared X slab
// in a dense item instead of one slab per block in runs (and the dense kernel multiplies every
// block of its grid, so it wants items at least half full); those columns go to dense items, TC
// at a time. Every other kept block goes to a run of its own row (TC_run columns at a time).
// Items with more blocks come first.
DwSchedule make_dw_items(const bsr_pattern &p) {
    const DwShape D = dw_dense_shape(p.b), Rn = dw_runs_shape(p.b);
    std::vector<std::pair<int32_t, std::vector<int32_t>>> dense, runs;   // (blocks, item)
    const std::vector<int32_t> rows = by_count_desc(p.row_ptr);
    std::vector<int32_t> pos(p.C, -1);   // CSR index of (row, column) for the current row
    std::vector<int32_t> count(p.C, 0);
    for (size_t g0 = 0; g0 < rows.size(); g0 += D.TR) {
        const int nr = (int)std::min<size_t>(D.TR, rows.size() - g0);
        std::fill(count.begin(), count.end(), 0);
        for (int i = 0; i < nr; ++i) {
            const int32_t r = rows[g0 + i];
            for (int32_t e = p.row_ptr[r]; e < p.row_ptr[r + 1]; ++e) count[p.col_idx[e]]++;
        }
        const int need = std::max(2, (nr + 1) / 2);
        std::vector<int32_t> dcols;
        for (int32_t c = 0; c < p.C; ++c)
            if (count[c] >= need) dcols.push_back(c);
        // dense items over the shared columns
        for (size_t c0 = 0; c0 < dcols.size(); c0 += D.TC) {
            const int nc = (int)std::min<size_t>(D.TC, dcols.size() - c0);
            std::vector<int32_t> it(D.TS(), -1);
            int nblk = 0;
            for (int i = 0; i < nr; ++i) it[i] = rows[g0 + i];
            for (int j = 0; j < nc; ++j) it[D.TR + j] = dcols[c0 + j];
            for (int i = 0; i < nr; ++i) {
                const int32_t r = rows[g0 + i];
                for (int32_t e = p.row_ptr[r]; e < p.row_ptr[r + 1]; ++e) pos[p.col_idx[e]] = e;
                for (int j = 0; j < nc; ++j) {
                    const int32_t e = pos[dcols[c0 + j]];
                    it[D.TR + D.TC + i * D.TC + j] = e;
                    nblk += e >= 0;
                }
                for (int32_t e = p.row_ptr[r]; e < p.row_ptr[r + 1]; ++e) pos[p.col_idx[e]] = -1;
            }
            dense.emplace_back(nblk, std::move(it));
        }
        // runs over the other blocks of each row
        for (int i = 0; i < nr; ++i) {
            const int32_t r = rows[g0 + i];
            std::vector<int32_t> rest;
            for (int32_t e = p.row_ptr[r]; e < p.row_ptr[r + 1]; ++e)
                if (count[p.col_idx[e]] < need) rest.push_back(e);
            for (size_t k0 = 0; k0 < rest.size(); k0 += Rn.TC) {
                const int nc = (int)std::min<size_t>(Rn.TC, rest.size() - k0);
                std::vector<int32_t> it(Rn.TS(), -1);
                it[0] = r;
                for (int j = 0; j < nc; ++j) {
                    it[1 + j] = p.col_idx[rest[k0 + j]];
                    it[1 + Rn.TC + j] = rest[k0 + j];
                }
                runs.emplace_back(nc, std::move(it));
            }
        }
    }
    auto pack = [](std::vector<std::pair<int32_t, std::vector<int32_t>>> &v) {
        std::stable_sort(v.begin(), v.end(), [](const auto &a, const auto &b) { return a.first > b.first; });
        DwItems out;
        out.n = (int)v.size();
        for (auto &x : v) out.items.insert(out.items.end(), x.second.begin(), x.second.end());
        return out;
    };
    DwSchedule s;
    s.dense = pack(dense);
    s.runs = pack(runs);
    // compact per-kind block numbering (for the split-M partial sums)
    s.cmap.assign(p.nnzb, -1);
    auto number = [&](const DwItems &v, int TS, int first_blk, int nblk, std::vector<int32_t> &list) {
        for (int k = 0; k < v.n; ++k)
            for (int q = 0; q < nblk; ++q) {
                const int32_t e = v.items[(size_t)k * TS + first_blk + q];
                if (e >= 0) {
                    s.cmap[e] = (int32_t)list.size();
                    list.push_back(e);
                }
            }
    };
    number(s.dense, D.TS(), D.TR + D.TC, D.TR * D.TC, s.dense_blocks);
    number(s.runs, Rn.TS(), Rn.TR + Rn.TC, Rn.TR * Rn.TC, s.run_blocks);
    return s;
}

}  // namespace

void build_pattern(bsr_pattern &p) {
    build_csc(p);
    const int G = gemm_group(p.b), S = gemm_slots(p.b, G);
    p.fwd = make_panels(p.row_ptr, p.col_idx, [](int32_t e) { return e; }, p.b, G, S);
    p.bwd = make_panels(p.col_ptr, p.row_idx, [&](int32_t e) { return p.perm[e]; }, p.b, G, S);
    p.dw = make_dw_items(p);
    p.rows_by_nnz = by_count_desc(p.row_ptr);
}

}  // namespace bsr
