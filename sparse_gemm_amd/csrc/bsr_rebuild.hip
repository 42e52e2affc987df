// bsr_rebuild.hip -- the pattern's CSR, CSC and perm metadata rebuilt on the device from a block
// mask, with no host round trip.
//
// The roadmap moves beyond patterns fixed at initialisation (pytorch_block_sparse summary page,
// "Future Development Roadmap"), and out-of-place mask updates let pruned weights grow back
// (pytorch/ao sparsity README, criteria list). When the mask changes during training, the index
// arrays can be rebuilt where the mask lives:
//   row counts and column counts (one work-group per row / per column),
//   exclusive scans into row_ptr and col_ptr (one work-group),
//   CSR fill: each row's kept columns in ascending order (a work-group-wide scan of the flags),
//   CSC fill: each column's kept rows in ascending order, with perm from the CSR position of every
//   kept block (a counting sort by column of the CSR entries, stable in the row).
// Integer work only, no atomics: the result is the canonical metadata, bit for bit.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "bsr_rebuild_internal.hpp"

namespace bsr {
namespace {

constexpr int kThreads = 256;

// Exclusive prefix of `flag` over the work-group (256 threads), and the work-group total.
__device__ __forceinline__ int wg_exclusive_scan(int flag, int *total, int *scratch /* [4] */) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const unsigned long long ballot = __ballot(flag);
    const int before = __popcll(ballot & ((1ull << lane) - 1ull));
    if (lane == 0) scratch[wave] = __popcll(ballot);
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) {
        const int c = scratch[w];
        off += w < wave ? c : 0;
        tot += c;
    }
    __syncthreads();   // scratch may be reused right after
    *total = tot;
    return off + before;
}

// Kept blocks of each row (work-group per row).
__global__ __launch_bounds__(kThreads) void k_row_counts(const uint8_t *__restrict__ mask, int C,
                                                         int32_t *__restrict__ cnt) {
    __shared__ int scratch[4];
    const int r = blockIdx.x;
    int n = 0;
    for (int c0 = 0; c0 < C; c0 += kThreads) {
        const int c = c0 + (int)threadIdx.x;
        int tot;
        (void)wg_exclusive_scan(c < C && mask[(int64_t)r * C + c] != 0, &tot, scratch);
        n += tot;
    }
    if (threadIdx.x == 0) cnt[r] = n;
}

// Kept blocks of each column (work-group per column); CAPPED: only those whose CSR position
// (pos, from k_fill_csr) lies below cap.
template <bool CAPPED>
__global__ __launch_bounds__(kThreads) void k_col_counts(const uint8_t *__restrict__ mask, int R, int C,
                                                         const int32_t *__restrict__ pos, int cap,
                                                         int32_t *__restrict__ cnt) {
    __shared__ int scratch[4];
    const int c = blockIdx.x;
    int n = 0;
    for (int r0 = 0; r0 < R; r0 += kThreads) {
        const int r = r0 + (int)threadIdx.x;
        int tot;
        const bool kept = r < R && mask[(int64_t)r * C + c] != 0;
        (void)wg_exclusive_scan(kept && (!CAPPED || pos[(int64_t)r * C + c] < cap), &tot, scratch);
        n += tot;
    }
    if (threadIdx.x == 0) cnt[c] = n;
}

// ptr[0] = 0, ptr[k + 1] = ptr[k] + cnt[k] for k < n (one work-group; each thread a contiguous
// segment); *total = ptr[n] when total is not null.
__global__ __launch_bounds__(kThreads) void k_scan(const int32_t *__restrict__ cnt, int n, int32_t *__restrict__ ptr,
                                                   int32_t *__restrict__ total) {
    __shared__ int part[kThreads];
    const int t = threadIdx.x;
    const int per = (n + kThreads - 1) / kThreads;
    const int b0 = min(n, t * per), b1 = min(n, b0 + per);
    int s = 0;
    for (int k = b0; k < b1; ++k) s += cnt[k];
    part[t] = s;
    __syncthreads();
    if (t == 0) {   // 256 partial sums, in order
        int run = 0;
        for (int k = 0; k < kThreads; ++k) {
            const int v = part[k];
            part[k] = run;
            run += v;
        }
    }
    __syncthreads();
    int run = part[t];
    for (int k = b0; k < b1; ++k) {
        ptr[k] = run;
        run += cnt[k];
    }
    if (t == kThreads - 1) {
        ptr[n] = run;
        if (total) *total = run;
    }
}

// CSR fill (work-group per row): col_idx in ascending column order; pos[r*C + c] = CSR position.
__global__ __launch_bounds__(kThreads) void k_fill_csr(const uint8_t *__restrict__ mask, int C,
                                                       const int32_t *__restrict__ row_ptr, int32_t *__restrict__ col_idx,
                                                       int cap, int32_t *__restrict__ pos) {
    __shared__ int scratch[4];
    const int r = blockIdx.x;
    int base = row_ptr[r];
    for (int c0 = 0; c0 < C; c0 += kThreads) {
        const int c = c0 + (int)threadIdx.x;
        const int flag = c < C && mask[(int64_t)r * C + c] != 0;
        int tot;
        const int j = base + wg_exclusive_scan(flag, &tot, scratch);
        if (flag) {
            pos[(int64_t)r * C + c] = j;
            if (j < cap) col_idx[j] = c;
        }
        base += tot;
    }
}

// CSC fill (work-group per column): row_idx in ascending row order, perm = CSR position; CAPPED:
// only the blocks whose CSR position lies below cap.
template <bool CAPPED>
__global__ __launch_bounds__(kThreads) void k_fill_csc(const uint8_t *__restrict__ mask, int R, int C,
                                                       const int32_t *__restrict__ col_ptr, const int32_t *__restrict__ pos,
                                                       int32_t *__restrict__ row_idx, int32_t *__restrict__ perm, int cap) {
    __shared__ int scratch[4];
    const int c = blockIdx.x;
    int base = col_ptr[c];
    for (int r0 = 0; r0 < R; r0 += kThreads) {
        const int r = r0 + (int)threadIdx.x;
        const bool kept = r < R && mask[(int64_t)r * C + c] != 0;
        const int flag = kept && (!CAPPED || pos[(int64_t)r * C + c] < cap);
        int tot;
        const int j = base + wg_exclusive_scan(flag, &tot, scratch);
        if (flag && j < cap) {
            row_idx[j] = r;
            perm[j] = pos[(int64_t)r * C + c];
        }
        base += tot;
    }
}

// ---- work lists of a device-built pattern ----
// The same record and item formats as the host-built lists (bsr_pattern.cpp), built by one thread
// per group (or per tile) in two passes over the device metadata: count, exclusive scan, fill.
// Groups take the output blocks in natural order (the host deals them heaviest first), which does
// not change any output: each output block still accumulates its kept blocks in ascending panel
// order. Positions at or past the capacity are dropped, as bsr_meta_rebuild drops them.

// Panel-GEMM records of group g: members g*G + t; entries e of member o in [ptr[o], min(ptr[o+1],
// cap)) have input block idx[e] and value block val(e) = e (forward) or perm[e] (input gradient;
// dropped when at or past cap). Returns the number of records; writes them at dst when not null.
template <int G, int S, int PB, bool CSC>
__device__ int group_records(int g, const int32_t *__restrict__ ptr, const int32_t *__restrict__ idx,
                            const int32_t *__restrict__ perm, int nout, int cap, int32_t *__restrict__ dst) {
    constexpr int U = G * PB;
    int cur[G], end[G];
#pragma unroll
    for (int t = 0; t < G; ++t) {
        const int o = g * G + t;
        cur[t] = o < nout ? min(ptr[o], cap) : 0;
        end[t] = o < nout ? min(ptr[o + 1], cap) : 0;
    }
    int nrec = 0;
    for (;;) {
        int panel = INT32_MAX;
#pragma unroll
        for (int t = 0; t < G; ++t)
            if (cur[t] < end[t]) panel = min(panel, idx[cur[t]] / PB);
        if (panel == INT32_MAX) break;
        int blk[U];
#pragma unroll
        for (int u = 0; u < U; ++u) blk[u] = -1;
#pragma unroll
        for (int t = 0; t < G; ++t)
            while (cur[t] < end[t] && idx[cur[t]] / PB == panel) {
                const int v = CSC ? perm[cur[t]] : cur[t];
                if (v >= 0 && v < cap) blk[t * PB + idx[cur[t]] % PB] = v;
                cur[t]++;
            }
        int u = 0;
        while (u < U) {
            int32_t r[kRecInts];
#pragma unroll
            for (int k = 0; k < kRecInts; ++k) r[k] = -1;
            r[0] = panel;
            uint32_t map[2] = {0xffffffffu, 0xffffffffu};
            int k = 0;
            for (; u < U && k < S; ++u) {
                if (blk[u] < 0) continue;
                r[1 + k] = blk[u];
                map[u / 8] &= ~(15u << (4 * (u % 8)));
                map[u / 8] |= (uint32_t)k << (4 * (u % 8));
                ++k;
            }
            if (k == 0) break;
            r[1 + S] = (int32_t)map[0];
            r[2 + S] = (int32_t)map[1];
            if (dst) {
#pragma unroll
                for (int q = 0; q < kRecInts; ++q) dst[(size_t)nrec * kRecInts + q] = r[q];
            }
            ++nrec;
        }
    }
    return nrec;
}

template <int G, int S, int PB, bool CSC>
__global__ __launch_bounds__(64) void k_group_count(const int32_t *__restrict__ ptr, const int32_t *__restrict__ idx,
                                                    const int32_t *__restrict__ perm, int nout, int cap,
                                                    int32_t *__restrict__ counts) {
    const int g = blockIdx.x * 64 + threadIdx.x;
    if (g >= (nout + G - 1) / G) return;
    counts[g] = group_records<G, S, PB, CSC>(g, ptr, idx, perm, nout, cap, nullptr);
}

template <int G, int S, int PB, bool CSC>
__global__ __launch_bounds__(64) void k_group_fill(const int32_t *__restrict__ ptr, const int32_t *__restrict__ idx,
                                                   const int32_t *__restrict__ perm, int nout, int cap,
                                                   const int32_t *__restrict__ sub_ptr, int32_t *__restrict__ rec,
                                                   int32_t *__restrict__ out, int32_t *__restrict__ order) {
    const int g = blockIdx.x * 64 + threadIdx.x;
    if (g >= (nout + G - 1) / G) return;
    (void)group_records<G, S, PB, CSC>(g, ptr, idx, perm, nout, cap, rec + (size_t)sub_ptr[g] * kRecInts);
    order[g] = g;
#pragma unroll
    for (int t = 0; t < G; ++t) out[g * G + t] = g * G + t < nout ? g * G + t : -1;
}

// First position in [lo, hi) of the ascending col_idx whose column is >= c.
__device__ __forceinline__ int lower_col(const int32_t *__restrict__ col_idx, int lo, int hi, int c) {
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (col_idx[mid] < c) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

// Weight-gradient items of tile t (TR x TC block positions at (r0, c0)): its kept blocks in row-major
// order, CAPI per item, each item's blocks spread over the kDwWaves compute waves in contiguous runs.
template <int TR, int TC, int CAPI>
__device__ int tile_items(int tile, const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ col_idx, int R,
                          int C, int cap, int32_t *__restrict__ dst) {
    const int ntc = (C + TC - 1) / TC;
    const int r0 = (tile / ntc) * TR, c0 = (tile % ntc) * TC;
    int n = 0;
    for (int r = r0; r < min(R, r0 + TR); ++r) {
        const int lo = min(row_ptr[r], cap), hi = min(row_ptr[r + 1], cap);
        n += lower_col(col_idx, lo, hi, c0 + TC) - lower_col(col_idx, lo, hi, c0);
    }
    const int nitems = (n + CAPI - 1) / CAPI;
    if (!dst) return nitems;
    int f = 0;   // running block number in the tile
    for (int r = r0; r < min(R, r0 + TR); ++r) {
        const int lo = min(row_ptr[r], cap), hi = min(row_ptr[r + 1], cap);
        const int e1 = lower_col(col_idx, lo, hi, c0 + TC);
        for (int e = lower_col(col_idx, lo, hi, c0); e < e1; ++e, ++f) {
            const int item = f / CAPI, q = f % CAPI;
            const int ni = min(CAPI, n - item * CAPI);   // blocks of this item
            int32_t *it = dst + (size_t)item * kDwItemInts;
            if (q == 0) {
                for (int k = 0; k < kDwItemInts; ++k) it[k] = 0;
                it[0] = r0;
                it[1] = c0;
                for (int w = 0; w < kDwWaves; ++w) it[2 + w] = ni * (w + 1) / kDwWaves - ni * w / kDwWaves;
            }
            int w = 0;
            while (ni * (w + 1) / kDwWaves <= q) ++w;   // the wave whose run holds block q
            const int q0 = ni * w / kDwWaves;
            it[16 + 8 * w + (q - q0)] = (int32_t)(((uint32_t)e << 8) | (uint32_t)((r - r0) << 4) | (uint32_t)(col_idx[e] - c0));
        }
    }
    return nitems;
}

template <int TR, int TC, int CAPI>
__global__ __launch_bounds__(64) void k_tile_count(const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ col_idx,
                                                   int R, int C, int cap, int32_t *__restrict__ counts) {
    const int t = blockIdx.x * 64 + threadIdx.x;
    if (t >= ((R + TR - 1) / TR) * ((C + TC - 1) / TC)) return;
    counts[t] = tile_items<TR, TC, CAPI>(t, row_ptr, col_idx, R, C, cap, nullptr);
}

template <int TR, int TC, int CAPI>
__global__ __launch_bounds__(64) void k_tile_fill(const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ col_idx,
                                                  int R, int C, int cap, const int32_t *__restrict__ item_ptr,
                                                  int32_t *__restrict__ items) {
    const int t = blockIdx.x * 64 + threadIdx.x;
    if (t >= ((R + TR - 1) / TR) * ((C + TC - 1) / TC)) return;
    (void)tile_items<TR, TC, CAPI>(t, row_ptr, col_idx, R, C, cap, items + (size_t)item_ptr[t] * kDwItemInts);
}

int32_t launched(const char *what) {
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return fail(BSR_ERR_HIP, std::string(what) + ": " + hipGetErrorString(err));
    return BSR_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

size_t rebuild_workspace_bytes(int32_t R, int32_t C) {
    return align256(sizeof(int32_t) * (size_t)R) + align256(sizeof(int32_t) * (size_t)C) +
           align256(sizeof(int32_t) * (size_t)R * (size_t)C);
}

int32_t launch_rebuild(int32_t R, int32_t C, const uint8_t *mask, int32_t *row_ptr, int32_t *col_idx,
                       int32_t *col_ptr, int32_t *row_idx, int32_t *perm, int32_t cap, int32_t *nnzb, void *ws,
                       void *stream, bool capped) {
    const hipStream_t st = (hipStream_t)stream;
    char *w = static_cast<char *>(ws);
    int32_t *rcnt = reinterpret_cast<int32_t *>(w);
    int32_t *ccnt = reinterpret_cast<int32_t *>(w + align256(sizeof(int32_t) * (size_t)R));
    int32_t *pos = reinterpret_cast<int32_t *>(w + align256(sizeof(int32_t) * (size_t)R) +
                                               align256(sizeof(int32_t) * (size_t)C));
    hipLaunchKernelGGL(k_row_counts, dim3((unsigned)R), dim3(kThreads), 0, st, mask, C, rcnt);
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(kThreads), 0, st, rcnt, R, row_ptr, nnzb);
    hipLaunchKernelGGL(k_fill_csr, dim3((unsigned)R), dim3(kThreads), 0, st, mask, C, row_ptr, col_idx, cap, pos);
    if (capped) {
        // the transposed lists hold exactly the blocks the CSR lists keep (CSR position below cap)
        hipLaunchKernelGGL(k_col_counts<true>, dim3((unsigned)C), dim3(kThreads), 0, st, mask, R, C, pos, cap, ccnt);
        hipLaunchKernelGGL(k_scan, dim3(1), dim3(kThreads), 0, st, ccnt, C, col_ptr, nullptr);
        hipLaunchKernelGGL(k_fill_csc<true>, dim3((unsigned)C), dim3(kThreads), 0, st, mask, R, C, col_ptr, pos, row_idx,
                           perm, cap);
    } else {
        hipLaunchKernelGGL(k_col_counts<false>, dim3((unsigned)C), dim3(kThreads), 0, st, mask, R, C, pos, cap, ccnt);
        hipLaunchKernelGGL(k_scan, dim3(1), dim3(kThreads), 0, st, ccnt, C, col_ptr, nullptr);
        hipLaunchKernelGGL(k_fill_csc<false>, dim3((unsigned)C), dim3(kThreads), 0, st, mask, R, C, col_ptr, pos, row_idx,
                           perm, cap);
    }
    return launched("metadata rebuild launch");
}

// Scratch of the work-list builders: group counts (forward, input gradient), tile item counts and
// their exclusive scan.
size_t sched_scratch_bytes(int32_t R, int32_t C, int b) {
    const int G = gemm_variant(b, kDeviceVariant).G;
    const int64_t ntiles = (int64_t)((R + dw_tile_rows(b) - 1) / dw_tile_rows(b)) * ((C + dw_tile_cols(b) - 1) / dw_tile_cols(b));
    return align256(sizeof(int32_t) * (size_t)((R + G - 1) / G)) + align256(sizeof(int32_t) * (size_t)((C + G - 1) / G)) +
           align256(sizeof(int32_t) * (size_t)ntiles) + align256(sizeof(int32_t) * (size_t)(ntiles + 1));
}

namespace {
template <int BS>
void launch_sched_bs(const bsr_pattern &p, hipStream_t st) {
    constexpr int G = BS == 32 ? 4 : 1, S = BS == 32 ? 4 : 1, PB = kPanelCols / BS;
    constexpr int TR = 256 / BS, TC = 512 / BS, CAPI = kDwWaves * (BS == 64 ? 2 : 8);
    static_assert(G * PB <= 8 && S < kRecInts - 2, "record layout");
    const DeviceMeta &d = p.dev;
    const DevSchedule &f = d.fwd[kDeviceVariant], &bw = d.bwd[kDeviceVariant];
    const int gf = (p.R + G - 1) / G, gb = (p.C + G - 1) / G;
    const int ntiles = ((p.R + TR - 1) / TR) * ((p.C + TC - 1) / TC);
    char *w = static_cast<char *>(d.sched_scratch);
    int32_t *cf = reinterpret_cast<int32_t *>(w);
    w += align256(sizeof(int32_t) * (size_t)gf);
    int32_t *cb = reinterpret_cast<int32_t *>(w);
    w += align256(sizeof(int32_t) * (size_t)gb);
    int32_t *ct = reinterpret_cast<int32_t *>(w);
    w += align256(sizeof(int32_t) * (size_t)ntiles);
    int32_t *item_ptr = reinterpret_cast<int32_t *>(w);
    const int cap = p.nnzb;
    auto blocks = [](int n) { return dim3((unsigned)((n + 63) / 64)); };
    auto mut = [](const int32_t *q) { return const_cast<int32_t *>(q); };
    // forward: groups of block rows over the CSR arrays
    hipLaunchKernelGGL((k_group_count<G, S, PB, false>), blocks(gf), dim3(64), 0, st, d.row_ptr, d.col_idx, d.perm,
                       p.R, cap, cf);
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(kThreads), 0, st, cf, gf, mut(f.sub_ptr), nullptr);
    hipLaunchKernelGGL((k_group_fill<G, S, PB, false>), blocks(gf), dim3(64), 0, st, d.row_ptr, d.col_idx, d.perm,
                       p.R, cap, f.sub_ptr, mut(f.rec), mut(f.out), mut(f.order));
    // input gradient: groups of block columns over the CSC arrays, value blocks through perm
    hipLaunchKernelGGL((k_group_count<G, S, PB, true>), blocks(gb), dim3(64), 0, st, d.col_ptr, d.row_idx, d.perm,
                       p.C, cap, cb);
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(kThreads), 0, st, cb, gb, mut(bw.sub_ptr), nullptr);
    hipLaunchKernelGGL((k_group_fill<G, S, PB, true>), blocks(gb), dim3(64), 0, st, d.col_ptr, d.row_idx, d.perm,
                       p.C, cap, bw.sub_ptr, mut(bw.rec), mut(bw.out), mut(bw.order));
    // weight gradient: tile items; their number goes to live_items
    hipLaunchKernelGGL((k_tile_count<TR, TC, CAPI>), blocks(ntiles), dim3(64), 0, st, d.row_ptr, d.col_idx, p.R, p.C,
                       cap, ct);
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(kThreads), 0, st, ct, ntiles, item_ptr, mut(d.live_items));
    hipLaunchKernelGGL((k_tile_fill<TR, TC, CAPI>), blocks(ntiles), dim3(64), 0, st, d.row_ptr, d.col_idx, p.R, p.C,
                       cap, item_ptr, mut(d.dw_items));
}
}  // namespace

// Rebuild of a device-built pattern from a device mask: the metadata, then the work lists.
int32_t launch_pattern_rebuild(const bsr_pattern &p, const uint8_t *mask, void *stream) {
    const DeviceMeta &d = p.dev;
    auto mut = [](const int32_t *q) { return const_cast<int32_t *>(q); };
    const int32_t rc = launch_rebuild(p.R, p.C, mask, mut(d.row_ptr), mut(d.col_idx), mut(d.col_ptr), mut(d.row_idx),
                                      mut(d.perm), p.nnzb, mut(d.live_nnzb), d.rebuild_ws, stream, true);
    if (rc != BSR_OK) return rc;
    const hipStream_t st = (hipStream_t)stream;
    if (p.b == 32) launch_sched_bs<32>(p, st);
    else launch_sched_bs<64>(p, st);
    return launched("work-list rebuild launch");
}

}  // namespace bsr
