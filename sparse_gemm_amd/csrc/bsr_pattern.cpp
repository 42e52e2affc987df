// bsr_pattern.cpp -- pattern metadata (CSR, transposed CSC + perm) and kernel work lists.
//
// Formats follow the pytorch/ao sparsity README, Table 4.1: BSR keeps dense blocks plus their
// coordinates; CSR / CSC keep an index pointer (where each row / column starts), the indices
// and the data. Blocks are canonical: ascending column inside a row, ascending row inside a
// column. The transposed form is what the input-gradient kernel walks, so it needs no atomics.
#include <algorithm>
#include <array>
#include <cstdlib>
#include <string>
#include <numeric>
#include <set>
#include <tuple>
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

// by_count_desc, equal counts ordered by their first input block (idx[ptr[o]], ascending; stable
// after that): output blocks with few kept blocks that share columns then share groups, so that a
// group walks fewer panels (Zipf 16384 x 4096 -> 11008 forward: 1188 -> 1074 sub-steps, the many
// single-block rows grouped by their column instead of by index)
std::vector<int32_t> by_count_desc_first(const std::vector<int32_t> &ptr, const std::vector<int32_t> &idx) {
    const int32_t n = (int32_t)ptr.size() - 1;
    std::vector<int32_t> ids(n);
    std::iota(ids.begin(), ids.end(), 0);
    auto first = [&](int32_t o) { return ptr[o + 1] > ptr[o] ? idx[ptr[o]] : INT32_MAX; };
    std::stable_sort(ids.begin(), ids.end(), [&](int32_t a, int32_t b) {
        const int32_t ca = ptr[a + 1] - ptr[a], cb = ptr[b + 1] - ptr[b];
        return ca != cb ? ca > cb : first(a) < first(b);
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
            ++s.npanels;
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

// Wide-tile schedule (b = 32): output blocks grouped kWideG at a time in order of decreasing
// kept-block count (so that rows with the same dense column set, e.g. full rows, share groups);
// each group walks the panels in which any member keeps a block, ascending, one sub-step each. A
// panel is two input blocks: `pairs[2p]`, `pairs[2p + 1]` (-1 = none), by default the consecutive
// blocks 2p, 2p + 1 (whole 128-byte lines of each activation row); the input gradient pairs the
// input blocks (block rows of W) in order of decreasing kept-block count instead, so that full
// rows share panels whose 16 units are all kept (Zipf 16384 x 4096 -> 11008: 1640 -> 1177
// sub-steps over the 16 groups).
template <class ValFn>
WideSchedule make_wide(const std::vector<int32_t> &ptr, const std::vector<int32_t> &idx, ValFn val, int32_t nin,
                       const std::vector<int32_t> &pairs) {
    constexpr int PB = kPanelCols / 32;
    const int32_t nout = (int32_t)ptr.size() - 1;
    const std::vector<int32_t> ids = by_count_desc_first(ptr, idx);
    // slot of each input block: panel * PB + unit half
    std::vector<int32_t> vin(nin, -1);
    for (size_t k = 0; k < pairs.size(); ++k)
        if (pairs[k] >= 0) vin[pairs[k]] = (int32_t)k;
    WideSchedule s;
    s.ngroups = (nout + kWideG - 1) / kWideG;
    s.out.assign((size_t)s.ngroups * kWideG, -1);
    s.sub_ptr.assign(s.ngroups + 1, 0);
    std::vector<std::vector<std::pair<int32_t, int32_t>>> ent(kWideG);   // (slot, value block), ascending
    std::vector<size_t> cursor(kWideG);
    for (int32_t g = 0; g < s.ngroups; ++g) {
        int members = 0;
        for (int t = 0; t < kWideG && g * kWideG + t < nout; ++t, ++members) {
            const int32_t o = ids[g * kWideG + t];
            s.out[(size_t)g * kWideG + t] = o;
            ent[t].clear();
            for (int32_t e = ptr[o]; e < ptr[o + 1]; ++e) ent[t].push_back({vin[idx[e]], val(e)});
            std::sort(ent[t].begin(), ent[t].end());
            cursor[t] = 0;
        }
        int32_t nsub = 0;
        for (;;) {
            int32_t panel = INT32_MAX;
            for (int t = 0; t < members; ++t)
                if (cursor[t] < ent[t].size()) panel = std::min(panel, ent[t][cursor[t]].first / PB);
            if (panel == INT32_MAX) break;
            std::vector<int32_t> r(kWideRecInts, 0);
            r[0] = panel;
            for (int u = 0; u < kWideU; ++u) r[2 + u] = -1;
            // the panel's two input blocks (a missing second one repeats the first: its units are
            // absent, so its staged bytes are never used)
            r[18] = pairs[(size_t)panel * PB];
            r[19] = pairs[(size_t)panel * PB + 1] >= 0 ? pairs[(size_t)panel * PB + 1] : r[18];
            uint32_t mask = 0;
            for (int t = 0; t < members; ++t)
                while (cursor[t] < ent[t].size() && ent[t][cursor[t]].first / PB == panel) {
                    const int u = t * PB + ent[t][cursor[t]].first % PB;
                    r[2 + u] = ent[t][cursor[t]].second;
                    mask |= 1u << u;
                    ++s.nunits;
                    cursor[t]++;
                }
            r[1] = (int32_t)mask;
            s.rec.insert(s.rec.end(), r.begin(), r.end());
            ++nsub;
        }
        s.sub_ptr[g + 1] = s.sub_ptr[g] + nsub;
    }
    s.flags.assign(s.ngroups, 0);
    for (int32_t g = 0; g < s.ngroups; ++g) {
        bool dense = s.sub_ptr[g + 1] > s.sub_ptr[g];
        for (int32_t k = s.sub_ptr[g]; k < s.sub_ptr[g + 1] && dense; ++k)
            dense = (uint32_t)s.rec[(size_t)k * kWideRecInts + 1] == (1u << kWideU) - 1;
        s.flags[g] = dense ? 1 : 0;
    }
    s.order.resize(s.ngroups);
    std::iota(s.order.begin(), s.order.end(), 0);
    std::stable_sort(s.order.begin(), s.order.end(), [&](int32_t a, int32_t b) {
        return s.sub_ptr[a + 1] - s.sub_ptr[a] > s.sub_ptr[b + 1] - s.sub_ptr[b];
    });
    return s;
}

// Consecutive input blocks in panels (2p, 2p + 1), padded with -1 to whole panels.
std::vector<int32_t> consecutive_pairs(int32_t nin) {
    std::vector<int32_t> v((size_t)(nin + 1) / 2 * 2, -1);
    for (int32_t k = 0; k < nin; ++k) v[k] = k;
    return v;
}

// Weight-gradient items: the kept blocks of every tile (dw_tile_rows x dw_tile_cols block
// positions) in row-major order, at most kDwWaves * dw_slots blocks per item (a fuller tile makes
// several items), spread over the compute waves in contiguous runs as even as possible (blocks of
// one run mostly share a row). Items are ordered by super-tiles of 8 x 4 tiles.
DwSchedule make_dw_items(const bsr_pattern &p, const std::vector<char> &taken) {
    const int TR = dw_tile_rows(p.b), TC = dw_tile_cols(p.b), SL = dw_slots(p.b), cap = kDwWaves * SL;
    std::vector<std::pair<int32_t, std::vector<int32_t>>> items;
    std::vector<int32_t> blk;   // (CSR index << 8) | (i << 4) | j, row-major inside the tile
    for (int32_t r0 = 0; r0 < p.R; r0 += TR) {
        for (int32_t c0 = 0; c0 < p.C; c0 += TC) {
            blk.clear();
            for (int32_t r = r0; r < std::min(p.R, r0 + TR); ++r)
                for (int32_t e = p.row_ptr[r]; e < p.row_ptr[r + 1]; ++e)
                    if (p.col_idx[e] >= c0 && p.col_idx[e] < c0 + TC && !taken[e])
                        blk.push_back((e << 8) | ((r - r0) << 4) | (p.col_idx[e] - c0));
            for (size_t f = 0; f < blk.size(); f += cap) {
                const int n = (int)std::min<size_t>(cap, blk.size() - f);
                std::vector<int32_t> it(kDwItemInts, 0);
                it[0] = r0;
                it[1] = c0;
                for (int w = 0; w < kDwWaves; ++w) {
                    const int q0 = n * w / kDwWaves, q1 = n * (w + 1) / kDwWaves;
                    it[2 + w] = q1 - q0;
                    for (int q = q0; q < q1; ++q) it[16 + 8 * w + (q - q0)] = blk[f + q];
                }
                items.emplace_back(n, std::move(it));
            }
        }
    }
    // super-tiles of 8 x 4 tiles (row-major), items of a tile in order: the kernel hands each XCD a
    // contiguous run of items, so the ones running together share dY and X row segments in L2
    auto key = [&](const std::vector<int32_t> &it) {
        return std::make_tuple(it[0] / (8 * TR), it[1] / (4 * TC), it[0], it[1]);
    };
    std::stable_sort(items.begin(), items.end(), [&](const auto &a, const auto &b) { return key(a.second) < key(b.second); });
    DwSchedule s;
    s.n = (int)items.size();
    for (auto &x : items) s.items.insert(s.items.end(), x.second.begin(), x.second.end());
    return s;
}

// Wide weight-gradient items (b = 32). Dense items first: block rows in order of decreasing kept-
// block count, 4 at a time, against every tile of 16 consecutive block columns that all 4 rows keep
// whole; they are ordered in runs of 8 row groups x 3 column tiles, so that the work-groups that run
// together on one XCD (a contiguous run of items) share activation column segments and gradient row
// segments in its L2. Then gathered items until every block is taken: the seed is the row with the
// most remaining blocks; with it go the 3 rows, among the next kWdwWindow by remaining count, that
// share most of its remaining columns (ties: more remaining blocks, then the order of the count
// list); the item takes the 16 columns that most of its rows keep (ties: lower column), in
// ascending column order; the blocks of gathered tiles that keep fewer than kWdwThinBelow go to thin
// items instead. Returns an empty schedule (every block left to the tile items) for b = 64
// and for patterns without a dense tile (measured: on BERT-base FFN-up and the square 10% layer the
// tile items take 25 and 83 us, the gathered wide items 31 and 94 us).
WideDwSchedule make_wide_dw(const bsr_pattern &p, std::vector<char> &taken) {
    WideDwSchedule s;
    taken.assign(p.nnzb, 0);
    if (p.b != 32 || p.nnzb == 0) return s;
    if (const char *f = std::getenv("BSR_DW_TILE"))   // tuning knob: 1 = tile items only
        if (std::atoi(f) == 1) return s;
    const int32_t R = p.R, C = p.C, W = (C + 63) / 64;
    std::vector<uint64_t> rem((size_t)R * W, 0);   // remaining (untaken) kept columns per row
    for (int32_t r = 0; r < R; ++r)
        for (int32_t e = p.row_ptr[r]; e < p.row_ptr[r + 1]; ++e)
            rem[(size_t)r * W + p.col_idx[e] / 64] |= uint64_t(1) << (p.col_idx[e] % 64);
    auto has = [&](int32_t r, int32_t c) { return (rem[(size_t)r * W + c / 64] >> (c % 64)) & 1; };
    auto csr = [&](int32_t r, int32_t c) {
        const auto b0 = p.col_idx.begin() + p.row_ptr[r], b1 = p.col_idx.begin() + p.row_ptr[r + 1];
        return (int32_t)(std::lower_bound(b0, b1, c) - p.col_idx.begin());
    };
    std::vector<std::vector<int32_t>> dense, gathered;
    auto make_item = [&](const std::vector<int32_t> &rows, const std::vector<int32_t> &cols) {
        std::vector<int32_t> it(kWdwItemInts, -1);
        for (size_t t = 0; t < rows.size(); ++t) it[t] = rows[t];
        for (size_t j = 0; j < cols.size(); ++j) it[4 + j] = cols[j];
        for (size_t t = 0; t < rows.size(); ++t)
            for (size_t j = 0; j < cols.size(); ++j)
                if (has(rows[t], cols[j])) {
                    const int32_t e = csr(rows[t], cols[j]);
                    it[kWdwBlockAt + 16 * t + j] = e;
                    taken[e] = 1;
                }
        for (size_t t = 0; t < rows.size(); ++t)
            for (size_t j = 0; j < cols.size(); ++j)
                if (it[kWdwBlockAt + 16 * t + j] >= 0)
                    rem[(size_t)rows[t] * W + cols[j] / 64] &= ~(uint64_t(1) << (cols[j] % 64));
        return it;
    };

    // dense items
    const std::vector<int32_t> order = by_count_desc(p.row_ptr);
    const int32_t ngr = R / kWdwRows, nct = C / kWdwCols;
    std::vector<std::vector<int32_t>> grid((size_t)ngr * nct);
    for (int32_t gr = 0; gr < ngr; ++gr) {
        const std::vector<int32_t> rows(order.begin() + gr * kWdwRows, order.begin() + (gr + 1) * kWdwRows);
        if (p.row_ptr[rows.back() + 1] - p.row_ptr[rows.back()] < kWdwCols) break;   // sorted: no more
        for (int32_t ct = 0; ct < nct; ++ct) {
            std::vector<int32_t> cols(kWdwCols);
            std::iota(cols.begin(), cols.end(), ct * kWdwCols);
            bool full = true;
            for (int32_t r : rows)
                for (int32_t c : cols) full = full && has(r, c);
            if (full) grid[(size_t)gr * nct + ct] = make_item(rows, cols);
        }
    }
    for (int32_t g0 = 0; g0 < ngr; g0 += 8)
        for (int32_t c0 = 0; c0 < nct; c0 += 3)
            for (int32_t ct = c0; ct < std::min(nct, c0 + 3); ++ct)
                for (int32_t gr = g0; gr < std::min(ngr, g0 + 8); ++gr)
                    if (!grid[(size_t)gr * nct + ct].empty()) dense.push_back(std::move(grid[(size_t)gr * nct + ct]));

    // gathered items over the remaining blocks; rows keyed by (remaining count desc, row asc)
    std::vector<int32_t> cnt(R, 0);
    std::set<std::pair<int32_t, int32_t>> live;
    for (int32_t r = 0; r < R; ++r) {
        for (int32_t w = 0; w < W; ++w) cnt[r] += __builtin_popcountll(rem[(size_t)r * W + w]);
        if (cnt[r]) live.insert({-cnt[r], r});
    }
    std::vector<int32_t> mult(C, 0);
    while (!live.empty()) {
        auto at = live.begin();
        const int32_t seed = at->second;
        struct Cand {
            int32_t shared, count, rank, row;
        };
        std::vector<Cand> cand;
        int32_t rank = 0;
        for (++at; at != live.end() && rank < kWdwWindow; ++at, ++rank) {
            int32_t sh = 0;
            for (int32_t w = 0; w < W; ++w)
                sh += __builtin_popcountll(rem[(size_t)seed * W + w] & rem[(size_t)at->second * W + w]);
            cand.push_back({sh, -at->first, rank, at->second});
        }
        std::sort(cand.begin(), cand.end(), [](const Cand &x, const Cand &y) {
            return std::make_tuple(-x.shared, -x.count, x.rank) < std::make_tuple(-y.shared, -y.count, y.rank);
        });
        std::vector<int32_t> rows = {seed};
        for (size_t k = 0; k < cand.size() && rows.size() < (size_t)kWdwRows; ++k) rows.push_back(cand[k].row);
        std::vector<int32_t> cols;
        for (int32_t r : rows)
            for (int32_t w = 0; w < W; ++w)
                for (uint64_t m = rem[(size_t)r * W + w]; m; m &= m - 1) {
                    const int32_t c = w * 64 + __builtin_ctzll(m);
                    if (mult[c]++ == 0) cols.push_back(c);
                }
        std::stable_sort(cols.begin(), cols.end(), [&](int32_t x, int32_t y) { return mult[x] != mult[y] ? mult[x] > mult[y] : x < y; });
        for (int32_t c : cols) mult[c] = 0;
        if (cols.size() > (size_t)kWdwCols) cols.resize(kWdwCols);
        std::sort(cols.begin(), cols.end());
        for (int32_t r : rows) live.erase({-cnt[r], r});
        gathered.push_back(make_item(rows, cols));
        for (int32_t r : rows) {
            cnt[r] = 0;
            for (int32_t w = 0; w < W; ++w) cnt[r] += __builtin_popcountll(rem[(size_t)r * W + w]);
            if (cnt[r]) live.insert({-cnt[r], r});
        }
    }
    if (dense.empty()) {   // no dense tile: the tile items do better (BERT-base FFN-up, the square layer)
        taken.assign(p.nnzb, 0);
        return s;
    }
    // gathered tiles keeping fewer than kWdwThinBelow blocks give them to thin items, by (column,
    // row): a 4 x 16 tile computes 64 products and stages 20 segments per step for its few blocks,
    // a thin item 1 product and 2 segments per block (Zipf layer: 52 of the 89 gathered tiles held
    // only rows with one block, 4 useful products of 64)
    std::vector<std::array<int32_t, 3>> pool;   // (column, row, CSR index)
    std::vector<std::vector<int32_t>> kept, thin;
    for (auto &it : gathered) {
        int cnt = 0;
        for (int k = 0; k < kWdwRows * kWdwCols; ++k) cnt += it[kWdwBlockAt + k] >= 0;
        if (cnt >= kWdwThinBelow) {
            kept.push_back(std::move(it));
            continue;
        }
        for (int t = 0; t < kWdwRows; ++t)
            for (int j = 0; j < kWdwCols; ++j)
                if (it[kWdwBlockAt + 16 * t + j] >= 0) pool.push_back({it[4 + j], it[t], it[kWdwBlockAt + 16 * t + j]});
    }
    gathered = std::move(kept);
    std::sort(pool.begin(), pool.end());
    for (size_t f = 0; f < pool.size(); f += kWdwThinBlocks) {
        std::vector<int32_t> it(kWdwItemInts, -1);
        it[kWdwKindAt] = 1;
        for (size_t k = 0; k < (size_t)kWdwThinBlocks && f + k < pool.size(); ++k) {
            it[4 + k] = pool[f + k][0];
            it[12 + k] = pool[f + k][1];
            it[kWdwBlockAt + k] = pool[f + k][2];
        }
        thin.push_back(std::move(it));
    }
    s.ndense = (int)dense.size();
    s.n = (int)(dense.size() + gathered.size() + thin.size());
    s.compact.assign(p.nnzb, -1);
    int32_t next = 0;
    for (auto *list : {&dense, &gathered, &thin})
        for (auto &it : *list) {
            s.first.push_back(next);
            for (int k = 0; k < kWdwRows * kWdwCols; ++k)
                if (it[kWdwBlockAt + k] >= 0) {
                    it[kWdwCompactAt + k] = next;
                    s.compact[next++] = it[kWdwBlockAt + k];
                }
            s.items.insert(s.items.end(), it.begin(), it.end());
        }
    s.first.push_back(next);
    return s;
}

}  // namespace

// Balanced small-M work list. A work item is up to two consecutive 16-row output slices of one block
// row; its bytes are the row's kept blocks times its slices. The items start as pairs of slices; the
// heaviest pairs are split into single slices until the count is a whole number of rounds of one item
// per compute unit (at most doubling it). Items are dealt heaviest first in the first round, lightest
// first in the second, and so on alternating, so that a unit's items balance each other (the
// work-groups of one launch are dealt to the units in order, round after round).
static std::vector<int32_t> small_m_work_list(const bsr_pattern &p) {
    struct Item {
        int64_t bytes;
        int32_t row, s0, ns;
    };
    const int S = p.b / 16;   // 16-row slices per block row
    std::vector<Item> items;
    for (int32_t r = 0; r < p.R; ++r)
        for (int s = 0; s < S; s += 2) items.push_back({(int64_t)(p.row_ptr[r + 1] - p.row_ptr[r]) * 2, r, s, 2});
    auto heavier = [](const Item &a, const Item &b) {
        return a.bytes != b.bytes ? a.bytes > b.bytes : a.row != b.row ? a.row < b.row : a.s0 < b.s0;
    };
    std::sort(items.begin(), items.end(), heavier);
    const size_t n = items.size();
    const size_t target = (n + kSmallMUnits - 1) / kSmallMUnits * kSmallMUnits;
    const size_t splits = std::min(n, target - n);
    std::vector<Item> all;
    for (size_t k = 0; k < n; ++k) {
        const Item &it = items[k];
        if (k < splits) {
            all.push_back({it.bytes / 2, it.row, it.s0, 1});
            all.push_back({it.bytes / 2, it.row, it.s0 + 1, 1});
        } else {
            all.push_back(it);
        }
    }
    std::sort(all.begin(), all.end(), heavier);
    for (size_t k0 = kSmallMUnits; k0 < all.size(); k0 += 2 * kSmallMUnits)
        std::reverse(all.begin() + k0, all.begin() + std::min(all.size(), k0 + kSmallMUnits));
    std::vector<int32_t> out;
    out.reserve(all.size() * 4);
    for (const Item &it : all) out.insert(out.end(), {it.row, p.row_ptr[it.row], p.row_ptr[it.row + 1], it.s0 | (it.ns << 8)});
    return out;
}

void csr_from_mask(int32_t R, int32_t C, const uint8_t *mask, std::vector<int32_t> &row_ptr,
                   std::vector<int32_t> &col_idx) {
    row_ptr.assign(R + 1, 0);
    col_idx.clear();
    for (int32_t r = 0; r < R; ++r) {
        for (int32_t c = 0; c < C; ++c)
            if (mask[(size_t)r * C + c]) col_idx.push_back(c);
        row_ptr[r + 1] = (int32_t)col_idx.size();
    }
}

const char *check_csr(int32_t R, int32_t C, int32_t nnzb, const int32_t *row_ptr, const int32_t *col_idx) {
    if (nnzb < 0 || (int64_t)nnzb > (int64_t)R * C) return "nnzb out of range";
    if (!row_ptr) return "row_ptr is NULL";
    if (nnzb > 0 && !col_idx) return "col_idx is NULL";
    if (row_ptr[0] != 0) return "row_ptr[0] must be 0";
    if (row_ptr[R] != nnzb) return "row_ptr[R] must equal nnzb";
    for (int32_t r = 0; r < R; ++r) {
        if (row_ptr[r + 1] < row_ptr[r]) return "row_ptr must be non-decreasing";
        if (row_ptr[r + 1] > nnzb) return "row_ptr exceeds nnzb";
        for (int32_t i = row_ptr[r]; i < row_ptr[r + 1]; ++i) {
            if (col_idx[i] < 0 || col_idx[i] >= C) return "col_idx out of range";
            if (i > row_ptr[r] && col_idx[i] <= col_idx[i - 1]) return "col_idx must be strictly increasing inside a row";
        }
    }
    return nullptr;
}

void build_pattern(bsr_pattern &p) {
    build_csc(p);
    for (int k = 0; k < kGemmVariants; ++k) {
        const GemmVariant v = gemm_variant(p.b, k);
        p.fwd[k] = make_panels(p.row_ptr, p.col_idx, [](int32_t e) { return e; }, p.b, v.G, v.S);
        p.bwd[k] = make_panels(p.col_ptr, p.row_idx, [&](int32_t e) { return p.perm[e]; }, p.b, v.G, v.S);
    }
    if (p.b == 32) {
        p.wide_fwd = make_wide(p.row_ptr, p.col_idx, [](int32_t e) { return e; }, p.C, consecutive_pairs(p.C));
        // input gradient: block rows of W paired by decreasing kept-block count, equal counts by
        // their first kept column (so rows with one block in the same column share a panel: Zipf
        // layer 1177 -> 1133 sub-steps by the host model)
        std::vector<int32_t> rows_pairs = by_count_desc_first(p.row_ptr, p.col_idx);
        if (const char *f = std::getenv("BSR_WIDE_PAIRS"))   // tuning knob: 0 = consecutive pairs
            if (std::atoi(f) == 0) rows_pairs = consecutive_pairs(p.R);
        rows_pairs.resize((size_t)(p.R + 1) / 2 * 2, -1);
        p.wide_bwd = make_wide(p.col_ptr, p.row_idx, [&](int32_t e) { return p.perm[e]; }, p.R, rows_pairs);
    } else {
        p.wide_fwd = WideSchedule();
        p.wide_bwd = WideSchedule();
    }
    std::vector<char> taken;
    p.wdw = make_wide_dw(p, taken);
    p.dw = make_dw_items(p, taken);
    // small-M forward row list (the fp8 and 2:4 forwards for few rows): one entry per block row,
    // {row, first block, end block, 0}. The rows of the first round of work-groups (one per compute
    // unit) come heaviest first and the rest lightest first, so that a unit's second work-group tends
    // to be a light one (decode shape, bf16 forward on this list: 14.44 -> 13.73 us against plain
    // heaviest-first).
    p.small_m_rows.clear();
    std::vector<int32_t> rows = by_count_desc(p.row_ptr);
    const size_t first = std::min(rows.size(), (size_t)(kSmallMUnits / std::max(1, p.b / 32)));
    std::reverse(rows.begin() + first, rows.end());
    for (int32_t r : rows) p.small_m_rows.insert(p.small_m_rows.end(), {r, p.row_ptr[r], p.row_ptr[r + 1], 0});
    p.small_m_work = small_m_work_list(p);
}

}  // namespace bsr
