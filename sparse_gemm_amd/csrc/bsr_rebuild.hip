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

// Kept blocks of each column (work-group per column).
__global__ __launch_bounds__(kThreads) void k_col_counts(const uint8_t *__restrict__ mask, int R, int C,
                                                         int32_t *__restrict__ cnt) {
    __shared__ int scratch[4];
    const int c = blockIdx.x;
    int n = 0;
    for (int r0 = 0; r0 < R; r0 += kThreads) {
        const int r = r0 + (int)threadIdx.x;
        int tot;
        (void)wg_exclusive_scan(r < R && mask[(int64_t)r * C + c] != 0, &tot, scratch);
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

// CSC fill (work-group per column): row_idx in ascending row order, perm = CSR position.
__global__ __launch_bounds__(kThreads) void k_fill_csc(const uint8_t *__restrict__ mask, int R, int C,
                                                       const int32_t *__restrict__ col_ptr, const int32_t *__restrict__ pos,
                                                       int32_t *__restrict__ row_idx, int32_t *__restrict__ perm, int cap) {
    __shared__ int scratch[4];
    const int c = blockIdx.x;
    int base = col_ptr[c];
    for (int r0 = 0; r0 < R; r0 += kThreads) {
        const int r = r0 + (int)threadIdx.x;
        const int flag = r < R && mask[(int64_t)r * C + c] != 0;
        int tot;
        const int j = base + wg_exclusive_scan(flag, &tot, scratch);
        if (flag && j < cap) {
            row_idx[j] = r;
            perm[j] = pos[(int64_t)r * C + c];
        }
        base += tot;
    }
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
                       void *stream) {
    const hipStream_t st = (hipStream_t)stream;
    char *w = static_cast<char *>(ws);
    int32_t *rcnt = reinterpret_cast<int32_t *>(w);
    int32_t *ccnt = reinterpret_cast<int32_t *>(w + align256(sizeof(int32_t) * (size_t)R));
    int32_t *pos = reinterpret_cast<int32_t *>(w + align256(sizeof(int32_t) * (size_t)R) +
                                               align256(sizeof(int32_t) * (size_t)C));
    hipLaunchKernelGGL(k_row_counts, dim3((unsigned)R), dim3(kThreads), 0, st, mask, C, rcnt);
    hipLaunchKernelGGL(k_col_counts, dim3((unsigned)C), dim3(kThreads), 0, st, mask, R, C, ccnt);
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(kThreads), 0, st, rcnt, R, row_ptr, nnzb);
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(kThreads), 0, st, ccnt, C, col_ptr, nullptr);
    hipLaunchKernelGGL(k_fill_csr, dim3((unsigned)R), dim3(kThreads), 0, st, mask, C, row_ptr, col_idx, cap, pos);
    hipLaunchKernelGGL(k_fill_csc, dim3((unsigned)C), dim3(kThreads), 0, st, mask, R, C, col_ptr, pos, row_idx, perm,
                       cap);
    return launched("metadata rebuild launch");
}

}  // namespace bsr
