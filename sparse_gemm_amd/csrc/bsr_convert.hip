// bsr_convert.hip -- dense <-> BSR conversion and block magnitudes on gfx950.
//
// The hand-off between a pruning front end and the sparse kernels is a dense weight with
// zeros in the dropped places (pytorch/ao sparsity README, workflow section); BSR keeps the
// dense blocks and their coordinates (README Table 4.1). The magnitude criterion keeps the
// blocks with the largest norm (README Table 4.2, L1 being the usual norm; pytorch_block_sparse
// summary page, "Future Development Roadmap": scoring parameter usefulness to choose the
// pattern).
//
// All three kernels are pure streams over HBM (each input byte read once, each output byte
// written once), so they are shaped for coalescing, not for the matrix cores:
//   k_block_norms     one work-group per (block row, 256-column strip): the strip is read in
//                     whole 512-byte row segments into LDS, one thread then sums one row of one
//                     block left to right in fp64, and the block's row sums are added in row
//                     order by one thread.
//   k_dense_to_values a fixed number of kept blocks per work-group; each 16-byte piece of a
//                     block is one load from the dense weight and one store into V.
//   k_values_to_dense one work-group per (block row, 256-column strip): the strip's kept
//                     blocks are found once in LDS, then every 16-byte piece of the strip is
//                     written exactly once (a block piece or zeros).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "bsr_convert_internal.hpp"

namespace bsr {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ double bf16_to_f64(uint32_t bits16) { return (double)__uint_as_float(bits16 << 16); }

// norms[r][c] = sum over p ascending of (sum over q ascending of t(W[r*BS+p][c*BS+q])), with
// t = |w| (KIND 1) or w*w (KIND 2), each sum left to right in fp64 from 0. The terms are exact in
// fp64 (a bf16 magnitude; a product of two 8-bit significands), and the order is fixed, so the
// result does not depend on the launch shape.
// Work-group = one block row x a strip of kNormCols columns (T = kNormCols / BS blocks). The strip
// is read with whole 512-byte row segments per 32 lanes (each byte once) into LDS; then thread
// (block j, row p) sums its row of block j from LDS, and T threads add the row sums in row order.
constexpr int kNormCols = 256;
constexpr int kNormLd = kNormCols + 8;   // LDS row stride in bf16: 16 bytes of padding per row

template <int BS, int KIND>
__global__ __launch_bounds__(256) void k_block_norms(const uint16_t *__restrict__ W, int K, int C,
                                                     double *__restrict__ norms) {
    constexpr int T = kNormCols / BS;             // blocks per strip (8 or 4); T * BS = 256 threads
    __shared__ __attribute__((aligned(16))) uint16_t tile[BS][kNormLd];
    __shared__ double rows[BS][T];
    const int t = threadIdx.x;
    const int r = blockIdx.y, c0 = blockIdx.x * T;
    const int ncols = min(kNormCols, (C - c0) * BS);   // columns of this strip inside W
    // phase 1: rows of the strip, 32 lanes x 16 bytes per row, 8 rows per pass
    const int seg = t & 31, prow = t >> 5;
#pragma unroll
    for (int k = 0; k < BS / 8; ++k) {
        const int p = k * 8 + prow;
        if (seg * 8 < ncols) {
            const u32x4 v = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4 *>(W + ((int64_t)r * BS + p) * K + (int64_t)c0 * BS + seg * 8));
            *reinterpret_cast<u32x4 *>(&tile[p][seg * 8]) = v;
        }
    }
    __syncthreads();
    // phase 2: thread (j, p) sums row p of block j left to right
    const int j = t % T, p = t / T;
    if (c0 + j < C) {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(&tile[p][j * BS]);
        double acc = 0.0;
#pragma unroll
        for (int q8 = 0; q8 < BS / 8; ++q8) {
            const u32x4 v = src[q8];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const double x = bf16_to_f64(e == 0 ? (v[h] & 0xffffu) : (v[h] >> 16));
                    if (KIND == 1)
                        acc += fabs(x);
                    else
                        acc += x * x;
                }
            }
        }
        rows[p][j] = acc;
    }
    __syncthreads();
    if (t < T && c0 + t < C) {
        double acc = 0.0;
#pragma unroll 8
        for (int q = 0; q < BS; ++q) acc += rows[q][t];
        norms[(int64_t)r * C + c0 + t] = acc;
    }
}

// Kept blocks per work-group of k_dense_to_values: 16 KB of block values each.
template <int BS>
constexpr int kGatherBlocks = 16384 / (2 * BS * BS);

// V[i][p][q] = W[r*BS + p][col_idx[i]*BS + q] for the kept blocks i of the work-group. The block
// row r of block i is found by a binary search of row_ptr (the last r with row_ptr[r] <= i).
template <int BS>
__global__ __launch_bounds__(256) void k_dense_to_values(const uint16_t *__restrict__ W, int K, int R,
                                                         const int32_t *__restrict__ row_ptr,
                                                         const int32_t *__restrict__ col_idx, int nnzb,
                                                         uint16_t *__restrict__ V) {
    constexpr int NB = kGatherBlocks<BS>;
    constexpr int PIECES = BS * BS / 8;          // 16-byte pieces per block
    constexpr int PER_THREAD = NB * PIECES / 256;
    __shared__ int64_t src_base[NB];
    const int t = threadIdx.x;
    const int i0 = blockIdx.x * NB;
    if (t < NB) {
        const int i = i0 + t;
        int64_t base = -1;
        if (i < nnzb) {
            int lo = 0, hi = R;  // row_ptr[lo] <= i < row_ptr[hi]
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (row_ptr[mid] <= i)
                    lo = mid;
                else
                    hi = mid;
            }
            base = (int64_t)lo * BS * K + (int64_t)col_idx[i] * BS;
        }
        src_base[t] = base;
    }
    __syncthreads();
    u32x4 v[PER_THREAD];
#pragma unroll
    for (int k = 0; k < PER_THREAD; ++k) {
        const int piece = k * 256 + t;
        const int lb = piece / PIECES, rem = piece % PIECES;
        const int p = rem / (BS / 8), q8 = rem % (BS / 8);
        const int64_t base = src_base[lb];
        if (base >= 0)
            v[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(W + base + (int64_t)p * K + q8 * 8));
    }
#pragma unroll
    for (int k = 0; k < PER_THREAD; ++k) {
        const int piece = k * 256 + t;
        const int lb = piece / PIECES;
        if (src_base[lb] >= 0)
            __builtin_nontemporal_store(v[k], reinterpret_cast<u32x4 *>(V + (int64_t)(i0 + lb) * BS * BS) +
                                                  (piece % PIECES));
    }
}

constexpr int kStripCols = 256;  // columns of the dense weight per work-group of k_values_to_dense

// The dense [N][K] weight: block (r, col_idx[i]) = V[i], zero elsewhere. Work-group (x, y) writes
// rows y*BS .. y*BS + BS - 1, columns x*256 .. x*256 + 255 (clipped at K).
template <int BS>
__global__ __launch_bounds__(256) void k_values_to_dense(const uint16_t *__restrict__ V, int K, int C,
                                                         const int32_t *__restrict__ row_ptr,
                                                         const int32_t *__restrict__ col_idx,
                                                         uint16_t *__restrict__ W) {
    constexpr int T = kStripCols / BS;            // block columns per strip
    constexpr int PER_THREAD = BS * (kStripCols / 8) / 256;
    __shared__ int32_t blk[T];
    const int t = threadIdx.x;
    const int r = blockIdx.y, c0 = blockIdx.x * T;
    if (t < T) blk[t] = -1;
    __syncthreads();
    const int e0 = row_ptr[r], e1 = row_ptr[r + 1];
    for (int e = e0 + t; e < e1; e += 256) {
        const int c = col_idx[e];
        if (c >= c0 && c < c0 + T) blk[c - c0] = e;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < PER_THREAD; ++k) {
        const int piece = k * 256 + t;
        const int p = piece / (kStripCols / 8), j = piece % (kStripCols / 8);
        const int lb = (j * 8) / BS, q = (j * 8) % BS;
        if (c0 + lb >= C) continue;
        const int i = blk[lb];
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (i >= 0) v = *reinterpret_cast<const u32x4 *>(V + ((int64_t)i * BS + p) * BS + q);
        __builtin_nontemporal_store(
            v, reinterpret_cast<u32x4 *>(W + ((int64_t)r * BS + p) * K + (int64_t)c0 * BS + j * 8));
    }
}

int32_t after_launch(const char *what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(BSR_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
    return BSR_OK;
}

}  // namespace

int32_t launch_block_norms(int32_t N, int32_t K, int32_t b, const uint16_t *W, int32_t kind, double *norms,
                           void *stream) {
    const int32_t R = N / b, C = K / b;
    if ((int64_t)R * C == 0) return BSR_OK;
    const int T = kNormCols / b;
    const dim3 grid((unsigned)((C + T - 1) / T), (unsigned)R);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (b == 32) {
        if (kind == 1)
            hipLaunchKernelGGL((k_block_norms<32, 1>), grid, dim3(256), 0, st, W, K, C, norms);
        else
            hipLaunchKernelGGL((k_block_norms<32, 2>), grid, dim3(256), 0, st, W, K, C, norms);
    } else {
        if (kind == 1)
            hipLaunchKernelGGL((k_block_norms<64, 1>), grid, dim3(256), 0, st, W, K, C, norms);
        else
            hipLaunchKernelGGL((k_block_norms<64, 2>), grid, dim3(256), 0, st, W, K, C, norms);
    }
    return after_launch("k_block_norms");
}

int32_t launch_dense_to_values(const bsr_pattern &p, const uint16_t *W, uint16_t *V, void *stream) {
    if (p.nnzb == 0) return BSR_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (p.b == 32) {
        const dim3 grid((unsigned)((p.nnzb + kGatherBlocks<32> - 1) / kGatherBlocks<32>));
        hipLaunchKernelGGL((k_dense_to_values<32>), grid, dim3(256), 0, st, W, p.K, p.R, p.dev.row_ptr,
                           p.dev.col_idx, p.nnzb, V);
    } else {
        const dim3 grid((unsigned)((p.nnzb + kGatherBlocks<64> - 1) / kGatherBlocks<64>));
        hipLaunchKernelGGL((k_dense_to_values<64>), grid, dim3(256), 0, st, W, p.K, p.R, p.dev.row_ptr,
                           p.dev.col_idx, p.nnzb, V);
    }
    return after_launch("k_dense_to_values");
}

int32_t launch_values_to_dense(const bsr_pattern &p, const uint16_t *V, uint16_t *W, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const unsigned strips = (unsigned)((p.K + kStripCols - 1) / kStripCols);
    const dim3 grid(strips, (unsigned)p.R);
    if (p.b == 32)
        hipLaunchKernelGGL((k_values_to_dense<32>), grid, dim3(256), 0, st, V, p.K, p.C, p.dev.row_ptr,
                           p.dev.col_idx, W);
    else
        hipLaunchKernelGGL((k_values_to_dense<64>), grid, dim3(256), 0, st, V, p.K, p.C, p.dev.row_ptr,
                           p.dev.col_idx, W);
    return after_launch("k_values_to_dense");
}

}  // namespace bsr
