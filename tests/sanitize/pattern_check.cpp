// Host half of the library under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only, built
// with g++ by tests/test_sanitizers.py): builds patterns from seeded block masks of many shapes and
// checks every invariant of the metadata and of the kernels' work lists, the rejection of malformed
// CSR, and the block-magnitude top-k. Prints "OK" and exits 0 when everything holds.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <numeric>
#include <vector>

#include "bsr_convert_internal.hpp"
#include "bsr_internal.hpp"

using namespace bsr;

static int g_fail = 0;
#define REQUIRE(c)                                                                  \
    do {                                                                            \
        if (!(c)) {                                                                 \
            std::fprintf(stderr, "%s:%d: %s failed\n", __FILE__, __LINE__, #c);      \
            if (++g_fail > 20) std::exit(1);                                        \
        }                                                                           \
    } while (0)

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd() {   // xorshift64*
    g_state ^= g_state >> 12;
    g_state ^= g_state << 25;
    g_state ^= g_state >> 27;
    return (uint32_t)((g_state * 0x2545F4914F6CDD1Dull) >> 32);
}

// A panel-GEMM schedule covers every kept block of its output blocks exactly once.
//   ptr/idx: output block -> input blocks (ascending); val(e) = value block of entry e.
template <class ValFn>
static void check_groups(const GroupSchedule &s, const std::vector<int32_t> &ptr, const std::vector<int32_t> &idx,
                         ValFn val, int b, int nvals) {
    const int PB = kPanelCols / b, U = s.G * PB;
    const int32_t nout = (int32_t)ptr.size() - 1;
    REQUIRE(s.ngroups == (nout + s.G - 1) / s.G);
    REQUIRE((int)s.sub_ptr.size() == s.ngroups + 1 && s.sub_ptr[0] == 0);
    REQUIRE((size_t)s.sub_ptr.back() * kRecInts == s.rec.size());
    std::vector<int> seen_out(nout, 0), seen_val(nvals, 0), seen_grp(s.ngroups, 0);
    for (int32_t g : s.order) {
        REQUIRE(g >= 0 && g < s.ngroups);
        if (g >= 0 && g < s.ngroups) seen_grp[g]++;
    }
    for (int g = 0; g < s.ngroups; ++g) REQUIRE(seen_grp[g] == 1);
    for (int g = 0; g < s.ngroups; ++g) {
        REQUIRE(s.sub_ptr[g + 1] >= s.sub_ptr[g]);
        int32_t last_panel = -1;
        for (int32_t k = s.sub_ptr[g]; k < s.sub_ptr[g + 1]; ++k) {
            const int32_t *r = &s.rec[(size_t)k * kRecInts];
            REQUIRE(r[0] >= last_panel);   // panels ascend
            last_panel = r[0];
            const uint32_t map[2] = {(uint32_t)r[1 + s.S], (uint32_t)r[2 + s.S]};
            int used = 0;
            for (int u = 0; u < U; ++u) {
                const int slot = (map[u / 8] >> (4 * (u % 8))) & 15;
                if (slot == 15) continue;
                REQUIRE(slot < s.S);
                ++used;
                const int t = u / PB;
                const int32_t o = s.out[(size_t)g * s.G + t];
                REQUIRE(o >= 0 && o < nout);
                if (o < 0 || o >= nout || slot >= s.S) continue;
                // the slot's value block is the member's block at input block panel * PB + u % PB
                const int32_t want_in = r[0] * PB + u % PB;
                int32_t e = -1;
                for (int32_t q = ptr[o]; q < ptr[o + 1]; ++q)
                    if (idx[q] == want_in) e = q;
                REQUIRE(e >= 0);
                if (e >= 0) {
                    REQUIRE(r[1 + slot] == val(e));
                    seen_val[val(e)]++;
                }
            }
            REQUIRE(used > 0 && used <= s.S);
            for (int k2 = used; k2 < s.S; ++k2) REQUIRE(r[1 + k2] == -1);
        }
        for (int t = 0; t < s.G; ++t) {
            const int32_t o = s.out[(size_t)g * s.G + t];
            if (o >= 0 && o < nout) seen_out[o]++;
        }
    }
    for (int32_t o = 0; o < nout; ++o) REQUIRE(seen_out[o] == 1);
    for (int v = 0; v < nvals; ++v) REQUIRE(seen_val[v] == 1);
}

static void check_pattern(const bsr_pattern &p) {
    const int32_t R = p.R, C = p.C, n = p.nnzb;
    // CSC + perm
    REQUIRE((int)p.col_ptr.size() == C + 1 && p.col_ptr[0] == 0 && p.col_ptr[C] == n);
    std::vector<int> hit(n, 0);
    for (int32_t c = 0; c < C; ++c) {
        REQUIRE(p.col_ptr[c + 1] >= p.col_ptr[c]);
        for (int32_t j = p.col_ptr[c]; j < p.col_ptr[c + 1]; ++j) {
            if (j > p.col_ptr[c]) REQUIRE(p.row_idx[j] > p.row_idx[j - 1]);
            const int32_t i = p.perm[j], r = p.row_idx[j];
            REQUIRE(i >= 0 && i < n && r >= 0 && r < R);
            if (i < 0 || i >= n || r < 0 || r >= R) continue;
            hit[i]++;
            REQUIRE(p.col_idx[i] == c && i >= p.row_ptr[r] && i < p.row_ptr[r + 1]);
        }
    }
    for (int32_t i = 0; i < n; ++i) REQUIRE(hit[i] == 1);
    // panel-GEMM work lists, forward (CSR) and input gradient (CSC)
    for (int k = 0; k < kGemmVariants; ++k) {
        const GemmVariant v = gemm_variant(p.b, k);
        REQUIRE(p.fwd[k].G == v.G && p.fwd[k].S == v.S && p.bwd[k].G == v.G && p.bwd[k].S == v.S);
        check_groups(p.fwd[k], p.row_ptr, p.col_idx, [](int32_t e) { return e; }, p.b, n);
        check_groups(p.bwd[k], p.col_ptr, p.row_idx, [&](int32_t e) { return p.perm[e]; }, p.b, n);
    }
    // wide panel-GEMM schedules (b = 32): one sub-step per panel any member keeps a block in;
    // every kept block once, at slot 2 t + (block % 2) of its member t; dense flags exact
    if (p.b == 32) {
        for (int dir = 0; dir < 2; ++dir) {
            const WideSchedule &s = dir ? p.wide_bwd : p.wide_fwd;
            const std::vector<int32_t> &ptr = dir ? p.col_ptr : p.row_ptr, &idx = dir ? p.row_idx : p.col_idx;
            const int32_t nout = (int32_t)ptr.size() - 1;
            REQUIRE(s.ngroups == (nout + kWideG - 1) / kWideG);
            REQUIRE((size_t)s.nsub() * kWideRecInts == s.rec.size() && (int)s.flags.size() == s.ngroups);
            std::vector<int> seen(n, 0), oseen(nout, 0);
            int64_t units = 0;
            std::vector<std::vector<std::pair<int32_t, int32_t>>> pair_of((size_t)(dir ? R : C) + 1);
            for (int g = 0; g < s.ngroups; ++g) {
                bool dense = s.sub_ptr[g + 1] > s.sub_ptr[g];
                for (int32_t k = s.sub_ptr[g]; k < s.sub_ptr[g + 1]; ++k) {
                    const int32_t *r = &s.rec[(size_t)k * kWideRecInts];
                    if (k > s.sub_ptr[g]) REQUIRE(r[0] > r[-kWideRecInts]);
                    dense = dense && (uint32_t)r[1] == 0xFFFFu;
                    REQUIRE(r[1] != 0);
                    // the panel's two input blocks: in range; the forward's are consecutive; a
                    // repeated first block (no second one) carries no unit of the second half
                    const int32_t nin = dir ? R : C;
                    REQUIRE(r[18] >= 0 && r[18] < nin && r[19] >= 0 && r[19] < nin);
                    if (!dir) REQUIRE(r[18] == 2 * r[0] && (r[19] == 2 * r[0] + 1 || (r[19] == r[18] && 2 * r[0] + 1 == C)));
                    if (r[19] == r[18])
                        for (int u = 1; u < kWideU; u += 2) REQUIRE(((r[1] >> u) & 1) == 0);
                    pair_of[(size_t)r[0]].push_back({r[18], r[19]});
                    for (int u = 0; u < kWideU; ++u) {
                        const bool present = (r[1] >> u) & 1;
                        REQUIRE(present == (r[2 + u] >= 0));
                        if (!present) continue;
                        const int32_t o = s.out[(size_t)g * kWideG + u / 2];
                        REQUIRE(o >= 0 && o < nout);
                        if (o < 0 || o >= nout) continue;
                        const int32_t want = u % 2 ? r[19] : r[18];
                        int32_t e = -1;
                        for (int32_t q = ptr[o]; q < ptr[o + 1]; ++q)
                            if (idx[q] == want) e = dir ? p.perm[q] : q;
                        REQUIRE(e >= 0 && r[2 + u] == e);
                        if (e >= 0) seen[e]++;
                        ++units;
                    }
                }
                REQUIRE(s.flags[g] == (dense ? 1 : 0));
                for (int t = 0; t < kWideG; ++t) {
                    const int32_t o = s.out[(size_t)g * kWideG + t];
                    if (o >= 0 && o < nout) oseen[o]++;
                }
            }
            REQUIRE(units == s.nunits && units == n);
            for (int32_t i = 0; i < n; ++i) REQUIRE(seen[i] == 1);
            for (int32_t o = 0; o < nout; ++o) REQUIRE(oseen[o] == 1);
            // one pair per panel, and every input block in at most one panel
            std::vector<int> in_panel((size_t)(dir ? R : C), 0);
            for (auto &v : pair_of) {
                for (auto &q : v) REQUIRE(q == v[0]);
                if (v.empty()) continue;
                in_panel[v[0].first]++;
                if (v[0].second != v[0].first) in_panel[v[0].second]++;
            }
            for (int x : in_panel) REQUIRE(x <= 1);
        }
    } else {
        REQUIRE(p.wide_fwd.ngroups == 0 && p.wide_bwd.ngroups == 0 && p.wdw.n == 0);
    }
    // weight-gradient items: every kept block exactly once over the wide items and the tile items
    // (no tile items once there are wide ones); a wide item's blocks are exactly the kept blocks of
    // its rows x columns that it claims, rows and columns distinct, dense items whole 4 x 16 tiles
    // of consecutive columns; compact indices number the blocks in item order
    const int TR = dw_tile_rows(p.b), TC = dw_tile_cols(p.b), SL = dw_slots(p.b);
    REQUIRE((size_t)p.dw.n * kDwItemInts == p.dw.items.size());
    REQUIRE((size_t)p.wdw.n * kWdwItemInts == p.wdw.items.size());
    if (p.wdw.n > 0) {
        REQUIRE(p.b == 32 && p.dw.n == 0);
        REQUIRE((int)p.wdw.compact.size() == n && (int)p.wdw.first.size() == p.wdw.n + 1);
        REQUIRE(p.wdw.ndense > 0 && p.wdw.ndense <= p.wdw.n);
    }
    std::fill(hit.begin(), hit.end(), 0);
    int32_t next = 0;
    bool seen_thin = false;
    for (int it = 0; it < p.wdw.n; ++it) {
        const int32_t *x = &p.wdw.items[(size_t)it * kWdwItemInts];
        REQUIRE(p.wdw.first[it] == next);
        // thin items (after every tile item): block k in column [4 + k], row [12 + k]; nothing else set
        REQUIRE(x[kWdwKindAt] == -1 || x[kWdwKindAt] == 1);
        if (x[kWdwKindAt] == 1) {
            seen_thin = true;
            REQUIRE(it >= p.wdw.ndense);
            int cnt = 0;
            for (int k = 0; k < kWdwItemInts; ++k) {
                const bool used = k == kWdwKindAt || (k >= 4 && k < 4 + kWdwThinBlocks) ||
                                  (k >= 12 && k < 12 + kWdwThinBlocks) ||
                                  (k >= kWdwBlockAt && k < kWdwBlockAt + kWdwThinBlocks) ||
                                  (k >= kWdwCompactAt && k < kWdwCompactAt + kWdwThinBlocks);
                if (!used) REQUIRE(x[k] == -1);
            }
            for (int k = 0; k < kWdwThinBlocks; ++k) {
                const int32_t e = x[kWdwBlockAt + k], c = x[kWdwCompactAt + k], col = x[4 + k], r = x[12 + k];
                REQUIRE((e >= 0) == (c >= 0) && (e >= 0) == (col >= 0) && (e >= 0) == (r >= 0));
                if (e < 0) continue;
                ++cnt;
                REQUIRE(e < n && r < R && col < C);
                if (e >= n || r >= R) continue;
                hit[e]++;
                REQUIRE(p.col_idx[e] == col && e >= p.row_ptr[r] && e < p.row_ptr[r + 1]);
                REQUIRE(c == next && p.wdw.compact[c] == e);
                ++next;
            }
            REQUIRE(cnt > 0);
            continue;
        }
        REQUIRE(!seen_thin);
        for (int t = 0; t < kWdwRows; ++t) {
            REQUIRE(x[t] >= -1 && x[t] < R);
            for (int u = 0; u < t; ++u) REQUIRE(x[t] < 0 || x[t] != x[u]);
        }
        for (int j = 0; j < kWdwCols; ++j) {
            REQUIRE(x[4 + j] >= -1 && x[4 + j] < C);
            for (int u = 0; u < j; ++u) REQUIRE(x[4 + j] < 0 || x[4 + j] != x[4 + u]);
        }
        const bool dense = it < p.wdw.ndense;
        int cnt = 0;
        for (int t = 0; t < kWdwRows; ++t)
            for (int j = 0; j < kWdwCols; ++j) {
                const int32_t e = x[kWdwBlockAt + 16 * t + j], c = x[kWdwCompactAt + 16 * t + j];
                REQUIRE((e >= 0) == (c >= 0));
                if (dense) REQUIRE(e >= 0 && x[4 + j] == x[4] + j && x[4] % kWdwCols == 0);
                if (e < 0) continue;
                ++cnt;
                const int32_t r = x[t], col = x[4 + j];
                REQUIRE(r >= 0 && col >= 0 && e < n);
                if (r < 0 || col < 0 || e >= n) continue;
                hit[e]++;
                REQUIRE(p.col_idx[e] == col && e >= p.row_ptr[r] && e < p.row_ptr[r + 1]);
                REQUIRE(c == next && p.wdw.compact[c] == e);
                ++next;
            }
        REQUIRE(cnt > 0);
    }
    if (p.wdw.n > 0) REQUIRE(p.wdw.first[p.wdw.n] == next && next == n);
    for (int it = 0; it < p.dw.n; ++it) {
        const int32_t *x = &p.dw.items[(size_t)it * kDwItemInts];
        const int32_t r0 = x[0], c0 = x[1];
        REQUIRE(r0 % TR == 0 && c0 % TC == 0 && r0 < R && c0 < C);
        for (int w = 0; w < kDwWaves; ++w) {
            REQUIRE(x[2 + w] >= 0 && x[2 + w] <= SL);
            for (int q = 0; q < x[2 + w] && q < SL; ++q) {
                const int32_t word = x[16 + 8 * w + q], e = word >> 8, i = (word >> 4) & 15, j = word & 15;
                REQUIRE(e >= 0 && e < n);
                if (e < 0 || e >= n) continue;
                hit[e]++;
                REQUIRE(p.col_idx[e] == c0 + j && e >= p.row_ptr[r0 + i] && e < p.row_ptr[r0 + i + 1]);
            }
        }
    }
    for (int32_t i = 0; i < n; ++i) REQUIRE(hit[i] == 1);
    // small-M lists: every block row once; the balanced list covers every 16-row slice once
    REQUIRE((int)p.small_m_rows.size() == 4 * R);
    std::vector<int> row_seen(R, 0);
    for (int32_t k = 0; k < R; ++k) {
        const int32_t r = p.small_m_rows[4 * k];
        REQUIRE(r >= 0 && r < R);
        if (r < 0 || r >= R) continue;
        row_seen[r]++;
        REQUIRE(p.small_m_rows[4 * k + 1] == p.row_ptr[r] && p.small_m_rows[4 * k + 2] == p.row_ptr[r + 1]);
    }
    for (int32_t r = 0; r < R; ++r) REQUIRE(row_seen[r] == 1);
    const int SLC = p.b / 16;
    std::vector<int> slice_seen((size_t)R * SLC, 0);
    REQUIRE(p.small_m_work.size() % 4 == 0);
    for (size_t k = 0; k + 3 < p.small_m_work.size(); k += 4) {
        const int32_t r = p.small_m_work[k], s0 = p.small_m_work[k + 3] & 0xff, ns = p.small_m_work[k + 3] >> 8;
        REQUIRE(r >= 0 && r < R && (ns == 1 || ns == 2) && s0 + ns <= SLC);
        if (r < 0 || r >= R || s0 + ns > SLC) continue;
        REQUIRE(p.small_m_work[k + 1] == p.row_ptr[r] && p.small_m_work[k + 2] == p.row_ptr[r + 1]);
        for (int q = s0; q < s0 + ns; ++q) slice_seen[(size_t)r * SLC + q]++;
    }
    for (size_t q = 0; q < slice_seen.size(); ++q) REQUIRE(slice_seen[q] == 1);
}

static void run_mask(int32_t R, int32_t C, int b, const std::vector<uint8_t> &mask) {
    bsr_pattern p;
    p.R = R;
    p.C = C;
    p.b = b;
    p.N = R * b;
    p.K = C * b;
    csr_from_mask(R, C, mask.data(), p.row_ptr, p.col_idx);
    p.nnzb = (int32_t)p.col_idx.size();
    REQUIRE(check_csr(R, C, p.nnzb, p.row_ptr.data(), p.col_idx.data()) == nullptr);
    int32_t count = 0;
    for (uint8_t m : mask) count += m != 0;
    REQUIRE(count == p.nnzb);
    build_pattern(p);
    check_pattern(p);
}

int main() {
    struct Shape {
        int32_t R, C;
        int b;
        double d;
    };
    const Shape shapes[] = {{1, 1, 32, 1.0}, {1, 1, 64, 0.0}, {8, 8, 32, 0.5},  {96, 24, 32, 0.25}, {128, 128, 32, 0.1},
                            {33, 7, 32, 0.9}, {7, 33, 32, 0.3}, {224, 64, 64, 0.5}, {40, 17, 64, 0.6}, {3, 700, 32, 0.05},
                            {600, 5, 32, 0.7}, {64, 64, 32, 1.0}, {17, 40, 32, 0.0}, {344, 128, 32, 0.3}};
    for (const Shape &sh : shapes) {
        std::vector<uint8_t> mask((size_t)sh.R * sh.C);
        for (auto &m : mask) m = (rnd() % 1000000) < (uint32_t)(sh.d * 1000000.0) ? 1 : 0;
        run_mask(sh.R, sh.C, sh.b, mask);
    }
    // uneven rows: a few full rows, many single-block rows, some empty ones (the Zipf case)
    {
        const int32_t R = 344, C = 128;
        std::vector<uint8_t> mask((size_t)R * C, 0);
        for (int32_t r = 0; r < R; ++r) {
            const uint32_t k = rnd() % 10;
            const int32_t cnt = k == 0 ? C : k < 6 ? 1 : k < 8 ? (int32_t)(rnd() % C) : 0;
            for (int32_t q = 0; q < cnt; ++q) mask[(size_t)r * C + rnd() % C] = 1;
        }
        run_mask(R, C, 32, mask);
    }
    // malformed CSR
    {
        const int32_t R = 3, C = 4;
        std::vector<int32_t> rp = {0, 2, 3, 5}, ci = {0, 2, 1, 0, 3};
        REQUIRE(check_csr(R, C, 5, rp.data(), ci.data()) == nullptr);
        std::vector<int32_t> bad;
        bad = {1, 2, 3, 5};
        REQUIRE(check_csr(R, C, 5, bad.data(), ci.data()) != nullptr);   // row_ptr[0] != 0
        bad = {0, 3, 2, 5};
        REQUIRE(check_csr(R, C, 5, bad.data(), ci.data()) != nullptr);   // decreasing
        bad = {0, 2, 3, 4};
        REQUIRE(check_csr(R, C, 5, bad.data(), ci.data()) != nullptr);   // row_ptr[R] != nnzb
        std::vector<int32_t> badc = {0, 2, 1, 0, 4};
        REQUIRE(check_csr(R, C, 5, rp.data(), badc.data()) != nullptr);  // column out of range
        badc = {0, 0, 1, 0, 3};
        REQUIRE(check_csr(R, C, 5, rp.data(), badc.data()) != nullptr);  // duplicate in a row
        badc = {2, 0, 1, 0, 3};
        REQUIRE(check_csr(R, C, 5, rp.data(), badc.data()) != nullptr);  // unsorted row
        REQUIRE(check_csr(R, C, 13, rp.data(), ci.data()) != nullptr);   // nnzb > R*C
        REQUIRE(check_csr(R, C, -1, rp.data(), ci.data()) != nullptr);
    }
    // top-k by block norm, ties to the lower index, against a full sort
    for (int trial = 0; trial < 20; ++trial) {
        const int32_t R = 1 + rnd() % 20, C = 1 + rnd() % 20;
        const int64_t n = (int64_t)R * C, keep = rnd() % (n + 1);
        std::vector<double> norms((size_t)n);
        for (auto &x : norms) x = (double)(rnd() % 7);   // many ties
        std::vector<uint8_t> mask((size_t)n, 2);
        REQUIRE(mask_topk(R, C, norms.data(), keep, mask.data()) == BSR_OK);
        std::vector<int64_t> idx((size_t)n);
        std::iota(idx.begin(), idx.end(), 0);
        std::stable_sort(idx.begin(), idx.end(), [&](int64_t a, int64_t b) { return norms[a] > norms[b]; });
        std::vector<uint8_t> want((size_t)n, 0);
        for (int64_t k = 0; k < keep; ++k) want[idx[k]] = 1;
        REQUIRE(mask == want);
    }
    if (g_fail) {
        std::fprintf(stderr, "%d checks failed\n", g_fail);
        return 1;
    }
    std::printf("OK\n");
    return 0;
}
