// bsr_kernels.hip -- gfx950 (CDNA4) kernels of the block-sparse linear layer.
//
// Every kept b x b block is a real dense contraction, so each one runs on bf16 MFMA with fp32
// accumulation (pytorch_block_sparse summary page, "Technical Foundation": dense matrix-core
// products on the kept blocks, zero blocks skipped). Output elements are rounded once to bf16.
//
// Operand layouts used below (CDNA4 bf16 MFMA, wave64):
//   v_mfma_f32_32x32x16_bf16: lane l holds A[l%32][8*(l/32) + t] and B[8*(l/32) + t][l%32],
//     t = 0..7; result item v of lane l is D[8*(v/4) + 4*(l/32) + v%4][l%32].
//   v_mfma_f32_16x16x32_bf16: lane l holds A[l%16][8*(l/16) + t] and B[8*(l/16) + t][l%16];
//     result item v of lane l is D[4*(l/16) + v][l%16].
// Only the pairing of A's and B's k positions matters for the sum, so both operands are
// always filled with the same k for the same (lane group, item).
//
// ds_read_tr16_b64 (transposing LDS read): in each group of 16 lanes, lane s supplies the
// address of 4 consecutive 16-bit values; lane i = 4u + v receives, as item t, value v of
// lane 4t + u. Pointing lane s at T[k0 + s/4][n0 + 4*(s%4)] of a row-major T[k][n] tile
// therefore hands lane i the four values T[k0..k0+3][n0 + i]: a k-run for one n, which is
// the MFMA operand layout for a tile stored n-contiguous.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "bsr_internal.hpp"

namespace bsr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kThreads = 256;  // 4 waves per work-group
constexpr int kTileM = 256;    // activation rows per work-group in the group GEMM (64 per wave)

__device__ __forceinline__ bf16x8 ld_global16(const uint16_t *p) { return *reinterpret_cast<const bf16x8 *>(p); }

__device__ __forceinline__ bf16x8 zero8() {
    i16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
    return __builtin_bit_cast(bf16x8, z);
}

// Two transposing LDS reads -> one 8-value MFMA operand: T[k0..k0+7][n0 + i] for lane i of
// its 16-lane group, where `row` points at T[k0] and `ld` is T's row pitch in elements.
__device__ __forceinline__ bf16x8 lds_read_tr8(const uint16_t *tile, int ld, int k0, int n0, int lane16) {
    const uint16_t *p0 = tile + (k0 + (lane16 >> 2)) * ld + n0 + 4 * (lane16 & 3);
    i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p0));
    i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p0 + 4 * ld));
    i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ uint16_t to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

__device__ __forceinline__ float from_bf16(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ void store4_bf16(uint16_t *dst, float a, float b, float c, float d) {
    const uint32_t lo = (uint32_t)to_bf16(a) | ((uint32_t)to_bf16(b) << 16);
    const uint32_t hi = (uint32_t)to_bf16(c) | ((uint32_t)to_bf16(d) << 16);
    *reinterpret_cast<uint2 *>(dst) = make_uint2(lo, hi);
}

// ------------------------------------------------------------------------------------------
// Group GEMM: forward (TRANS = false) and input gradient (TRANS = true).
//
// Work-group = (group of G output blocks, 256 activation rows). Output blocks are block rows
// of W for the forward (out = Y, act = X) and block columns for the input gradient (out = dX,
// act = dY, walking the transposed metadata). Each step takes one input block of the
// activations (block column c of X, or block row r of dY) and the value blocks of the group's
// members that sit there. Per wave: 64 activation rows; per member: a BS x 64 output tile
// computed as (weight block) x (activations)^T, so each lane ends up holding 4 consecutive
// output columns of one activation row.
//   forward:  A[n][k] = V[i][n][k]                  (natural layout, 16-byte LDS reads)
//   input grad: A[n][k] = V[i][k][n] (transposed)   (ds_read_tr16_b64 of the natural layout)
//   B[k][m] = act[m][in*BS + k]                     (16-byte global loads)
// ------------------------------------------------------------------------------------------
template <int BS, int G, bool TRANS>
__global__ __launch_bounds__(kThreads) void k_group_gemm(
    const uint16_t *__restrict__ act, int in_ld, int64_t M, const uint16_t *__restrict__ V,
    const uint16_t *__restrict__ bias, uint16_t *__restrict__ out, int out_ld, const int32_t *__restrict__ order,
    const int32_t *__restrict__ step_ptr, const int32_t *__restrict__ gout, const int32_t *__restrict__ step_in,
    const int32_t *__restrict__ step_blk, int nmtiles) {
    constexpr int NS = BS / 32;   // 32-row slices of a block
    constexpr int KK = BS / 16;   // 16-wide k chunks of a block
    constexpr int LDW = BS + 8;   // padded LDS pitch (elements)
    constexpr int CH = BS * BS / 8;  // 16-byte chunks per block
    __shared__ __attribute__((aligned(16))) uint16_t wl[G][BS][LDW];

    const int g = order[blockIdx.x / nmtiles];
    const int mt = blockIdx.x % nmtiles;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t mbase = (int64_t)mt * kTileM + wave * 64;

    f32x16 acc[G][NS][2];
#pragma unroll
    for (int t = 0; t < G; ++t)
#pragma unroll
        for (int ns = 0; ns < NS; ++ns)
#pragma unroll
            for (int ms = 0; ms < 2; ++ms)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[t][ns][ms][v] = 0.f;

    const int s0 = step_ptr[g], s1 = step_ptr[g + 1];
    for (int s = s0; s < s1; ++s) {
        const int in_blk = step_in[s];
        bf16x8 bfr[2][KK];
#pragma unroll
        for (int ms = 0; ms < 2; ++ms) {
            const int64_t m = mbase + ms * 32 + (lane & 31);
            const uint16_t *src = act + m * in_ld + (int64_t)in_blk * BS + (lane >> 5) * 8;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) bfr[ms][kk] = (m < M) ? ld_global16(src + kk * 16) : zero8();
        }
        __syncthreads();  // the previous step's LDS reads are done
        for (int e = threadIdx.x; e < G * CH; e += kThreads) {
            const int t = e / CH, w = e % CH;
            const int blk = step_blk[s * G + t];
            if (blk >= 0) {
                const int row = w / (BS / 8), c8 = (w % (BS / 8)) * 8;
                *reinterpret_cast<uint4 *>(&wl[t][row][c8]) =
                    *reinterpret_cast<const uint4 *>(V + (size_t)blk * BS * BS + row * BS + c8);
            }
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < G; ++t) {
            if (step_blk[s * G + t] < 0) continue;  // uniform over the work-group
#pragma unroll
            for (int ns = 0; ns < NS; ++ns) {
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    bf16x8 a;
                    if constexpr (!TRANS) {
                        a = *reinterpret_cast<const bf16x8 *>(&wl[t][ns * 32 + (lane & 31)][kk * 16 + (lane >> 5) * 8]);
                    } else {
                        const int gq = lane >> 4;
                        a = lds_read_tr8(&wl[t][0][0], LDW, kk * 16 + (gq >> 1) * 8, ns * 32 + (gq & 1) * 16, lane & 15);
                    }
#pragma unroll
                    for (int ms = 0; ms < 2; ++ms)
                        acc[t][ns][ms] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bfr[ms][kk], acc[t][ns][ms], 0, 0, 0);
                }
            }
        }
    }

    // Epilogue: item v of lane l is output column 8*(v/4) + 4*(l/32) + v%4 of the 32-column
    // slice, activation row l%32 of the 32-row slice.
#pragma unroll
    for (int t = 0; t < G; ++t) {
        const int o = gout[g * G + t];
        if (o < 0) continue;
#pragma unroll
        for (int ms = 0; ms < 2; ++ms) {
            const int64_t m = mbase + ms * 32 + (lane & 31);
            if (m >= M) continue;
#pragma unroll
            for (int ns = 0; ns < NS; ++ns) {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int n = o * BS + ns * 32 + q4 * 8 + (lane >> 5) * 4;
                    float v0 = acc[t][ns][ms][q4 * 4 + 0], v1 = acc[t][ns][ms][q4 * 4 + 1];
                    float v2 = acc[t][ns][ms][q4 * 4 + 2], v3 = acc[t][ns][ms][q4 * 4 + 3];
                    if (bias) {
                        const uint2 bb = *reinterpret_cast<const uint2 *>(bias + n);
                        v0 += from_bf16(bb.x & 0xffff);
                        v1 += from_bf16(bb.x >> 16);
                        v2 += from_bf16(bb.y & 0xffff);
                        v3 += from_bf16(bb.y >> 16);
                    }
                    store4_bf16(out + m * out_ld + n, v0, v1, v2, v3);
                }
            }
        }
    }
}

// ------------------------------------------------------------------------------------------
// Small-M forward (M <= 16): a streaming pass over the block values ("load sparse, expand,
// dense MMA" for memory-bound shapes, GPU MODE lecture 11 summary at 48:12). One wave per
// (block row, 16-row slice of the block): it reads that slice of every kept block of the row
// once (16 contiguous rows of BS values) and multiplies it with the matching X columns.
//   A[p][k] = V[i][slice*16 + p][k]   B[k][m] = X[m][c*BS + k]   (16x16x32 MFMA, m < 16)
// Output rows p of the slice are disjoint between waves, so no reduction is needed.
// ------------------------------------------------------------------------------------------
template <int BS>
__global__ __launch_bounds__(64) void k_small_m(const uint16_t *__restrict__ X, int K, int M,
                                                const uint16_t *__restrict__ V, const uint16_t *__restrict__ bias,
                                                uint16_t *__restrict__ Y, int N, const int32_t *__restrict__ row_ptr,
                                                const int32_t *__restrict__ col_idx,
                                                const int32_t *__restrict__ rows_by_nnz) {
    constexpr int PS = BS / 16;  // 16-row slices per block
    constexpr int KC = BS / 32;  // 32-wide k chunks per block
    constexpr int U = 4;         // blocks in flight per wave
    const int r = rows_by_nnz[blockIdx.x / PS];
    const int slice = blockIdx.x % PS;
    const int lane = threadIdx.x;
    const int m = lane & 15;
    const bool mvalid = m < M;
    const int kofs = (lane >> 4) * 8;
    const uint16_t *vrow = V + (size_t)(slice * 16 + (lane & 15)) * BS + kofs;
    const uint16_t *xrow = X + (int64_t)(mvalid ? m : 0) * K + kofs;

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int i0 = row_ptr[r], i1 = row_ptr[r + 1];
    int i = i0;
    for (; i + U <= i1; i += U) {
        bf16x8 a[U][KC], b[U][KC];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = col_idx[i + u];
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                a[u][kc] = ld_global16(vrow + (size_t)(i + u) * BS * BS + kc * 32);
                b[u][kc] = mvalid ? ld_global16(xrow + (int64_t)c * BS + kc * 32) : zero8();
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][kc], b[u][kc], acc, 0, 0, 0);
    }
    for (; i < i1; ++i) {
        const int c = col_idx[i];
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            bf16x8 a = ld_global16(vrow + (size_t)i * BS * BS + kc * 32);
            bf16x8 b = mvalid ? ld_global16(xrow + (int64_t)c * BS + kc * 32) : zero8();
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
        }
    }
    if (mvalid) {
        const int n = r * BS + slice * 16 + (lane >> 4) * 4;
        float v0 = acc[0], v1 = acc[1], v2 = acc[2], v3 = acc[3];
        if (bias) {
            const uint2 bb = *reinterpret_cast<const uint2 *>(bias + n);
            v0 += from_bf16(bb.x & 0xffff);
            v1 += from_bf16(bb.x >> 16);
            v2 += from_bf16(bb.y & 0xffff);
            v3 += from_bf16(bb.y >> 16);
        }
        store4_bf16(Y + (int64_t)m * N + n, v0, v1, v2, v3);
    }
}

// ------------------------------------------------------------------------------------------
// Weight gradient on the kept blocks (block-masked SDDMM): for block i of row r, column c,
//   dV[i][p][q] = sum_m dY[m][r*BS + p] * X[m][c*BS + q].
// Work-group = (block i, chunk of M). Both operands have the reduction index m as their slow
// index in memory, so 64-row slabs of dY[:, r-block] and X[:, c-block] are staged in LDS in
// their natural layout and read back transposed with ds_read_tr16_b64.
//   BS = 32: wave w owns the 16 x 16 output tile w (16x16x32 MFMA).
//   BS = 64: wave w owns the 32 x 32 output tile w (32x32x16 MFMA).
// With one chunk the result is rounded to bf16 directly; otherwise fp32 partials go to the
// workspace and k_dw_reduce sums them in chunk order.
// ------------------------------------------------------------------------------------------
template <int BS>
__global__ __launch_bounds__(kThreads) void k_dw(const uint16_t *__restrict__ dY, int N,
                                                 const uint16_t *__restrict__ X, int K, int64_t M,
                                                 const int32_t *__restrict__ blk_row,
                                                 const int32_t *__restrict__ col_idx, int64_t mchunk, int nchunks,
                                                 int nnzb, float *__restrict__ partial, uint16_t *__restrict__ dV) {
    constexpr int SLAB = 64;
    constexpr int LDS_LD = BS + 8;
    constexpr int CPR = BS / 8;  // 16-byte chunks per slab row
    __shared__ __attribute__((aligned(16))) uint16_t sdy[SLAB][LDS_LD];
    __shared__ __attribute__((aligned(16))) uint16_t sx[SLAB][LDS_LD];

    const int i = blockIdx.x / nchunks;
    const int ch = blockIdx.x % nchunks;
    const int r = blk_row[i], c = col_idx[i];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t m_begin = (int64_t)ch * mchunk;
    const int64_t m_end = std::min<int64_t>(M, m_begin + mchunk);

    constexpr int TD = (BS == 32) ? 16 : 32;     // output tile edge per wave
    const int p0 = (wave >> 1) * TD, q0 = (wave & 1) * TD;
    f32x16 acc32 = {};
    f32x4 acc16 = {0.f, 0.f, 0.f, 0.f};

    for (int64_t ms = m_begin; ms < m_end; ms += SLAB) {
        __syncthreads();
        for (int e = threadIdx.x; e < 2 * SLAB * CPR; e += kThreads) {
            const int which = e / (SLAB * CPR);
            const int w = e % (SLAB * CPR);
            const int row = w / CPR, c8 = (w % CPR) * 8;
            const int64_t m = ms + row;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (m < m_end) {
                const uint16_t *src = which ? (X + m * K + (int64_t)c * BS + c8) : (dY + m * N + (int64_t)r * BS + c8);
                v = *reinterpret_cast<const uint4 *>(src);
            }
            uint16_t *dst = which ? &sx[row][c8] : &sdy[row][c8];
            *reinterpret_cast<uint4 *>(dst) = v;
        }
        __syncthreads();
        if constexpr (BS == 32) {
            // A[p][m] = sdy[m][p0 + p], B[m][q] = sx[m][q0 + q]; k = m, 32 per MFMA
            const int gq = lane >> 4;
#pragma unroll
            for (int kc = 0; kc < SLAB / 32; ++kc) {
                const bf16x8 a = lds_read_tr8(&sdy[0][0], LDS_LD, kc * 32 + gq * 8, p0, lane & 15);
                const bf16x8 b = lds_read_tr8(&sx[0][0], LDS_LD, kc * 32 + gq * 8, q0, lane & 15);
                acc16 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc16, 0, 0, 0);
            }
        } else {
            // 32x32x16: lane group gq covers rows/cols (gq&1)*16.., k = (gq>>1)*8..
            const int gq = lane >> 4;
#pragma unroll
            for (int kc = 0; kc < SLAB / 16; ++kc) {
                const bf16x8 a = lds_read_tr8(&sdy[0][0], LDS_LD, kc * 16 + (gq >> 1) * 8, p0 + (gq & 1) * 16, lane & 15);
                const bf16x8 b = lds_read_tr8(&sx[0][0], LDS_LD, kc * 16 + (gq >> 1) * 8, q0 + (gq & 1) * 16, lane & 15);
                acc32 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc32, 0, 0, 0);
            }
        }
    }

    // write the tile: (p, q) pairs per lane from the MFMA result layout
    const size_t blk_off = (size_t)i * BS * BS;
    if constexpr (BS == 32) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int p = p0 + (lane >> 4) * 4 + v, q = q0 + (lane & 15);
            if (nchunks == 1) dV[blk_off + p * BS + q] = to_bf16(acc16[v]);
            else partial[((size_t)ch * nnzb) * BS * BS + blk_off + p * BS + q] = acc16[v];
        }
    } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int p = p0 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3), q = q0 + (lane & 31);
            if (nchunks == 1) dV[blk_off + p * BS + q] = to_bf16(acc32[v]);
            else partial[((size_t)ch * nnzb) * BS * BS + blk_off + p * BS + q] = acc32[v];
        }
    }
}

// Sums the per-chunk fp32 partials in chunk order and rounds to bf16.
__global__ __launch_bounds__(kThreads) void k_dw_reduce(const float *__restrict__ partial, int nchunks, size_t count,
                                                        uint16_t *__restrict__ dV) {
    const size_t e = (size_t)blockIdx.x * kThreads + threadIdx.x;
    if (e >= count) return;
    float s = 0.f;
    for (int ch = 0; ch < nchunks; ++ch) s += partial[(size_t)ch * count + e];
    dV[e] = to_bf16(s);
}

// Bias gradient, pass 1: column sums of dY over one chunk of rows -> fp32 partials.
__global__ __launch_bounds__(kThreads) void k_colsum_partial(const uint16_t *__restrict__ dY, int N, int64_t M,
                                                             int64_t rows_per, float *__restrict__ partial) {
    const int n = blockIdx.x * kThreads + threadIdx.x;
    const int ch = blockIdx.y;
    if (n >= N) return;
    const int64_t m0 = (int64_t)ch * rows_per, m1 = std::min<int64_t>(M, m0 + rows_per);
    float s = 0.f;
    for (int64_t m = m0; m < m1; ++m) s += from_bf16(dY[m * N + n]);
    partial[(size_t)ch * N + n] = s;
}

// Bias gradient, pass 2: sum the partials in chunk order.
__global__ __launch_bounds__(kThreads) void k_colsum_final(const float *__restrict__ partial, int nchunks, int N,
                                                           uint16_t *__restrict__ db) {
    const int n = blockIdx.x * kThreads + threadIdx.x;
    if (n >= N) return;
    float s = 0.f;
    for (int ch = 0; ch < nchunks; ++ch) s += partial[(size_t)ch * N + n];
    db[n] = to_bf16(s);
}

__global__ __launch_bounds__(kThreads) void k_fill_zero(uint16_t *__restrict__ p, size_t count) {
    const size_t e = (size_t)blockIdx.x * kThreads + threadIdx.x;
    if (e < count) p[e] = 0;
}

// ---- host-side sizing shared by the workspace query and the launcher ----
struct DwPlan {
    int nchunks = 1;
    int64_t mchunk = 0;
    int bchunks = 1;        // row chunks of the bias column sums
    int64_t brows = 0;
    size_t partial_off = 0, partial_bytes = 0, bias_off = 0, bias_bytes = 0, total = 0;
};

DwPlan plan_dw(const bsr_pattern &p, int64_t M) {
    DwPlan d;
    if (M <= 0) return d;
    // enough work-groups to cover the chip twice, without chunks shorter than 256 rows
    const int64_t want = std::max<int64_t>(1, (2048 + std::max(p.nnzb, 1) - 1) / std::max(p.nnzb, 1));
    const int64_t maxc = std::max<int64_t>(1, M / 256);
    d.nchunks = (int)std::min<int64_t>(want, maxc);
    d.mchunk = ((M + d.nchunks - 1) / d.nchunks + 63) / 64 * 64;
    d.nchunks = (int)((M + d.mchunk - 1) / d.mchunk);
    d.bchunks = (int)std::min<int64_t>(64, std::max<int64_t>(1, M / 256));
    d.brows = (M + d.bchunks - 1) / d.bchunks;
    d.bchunks = (int)((M + d.brows - 1) / d.brows);
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    d.partial_bytes = d.nchunks > 1 ? (size_t)d.nchunks * p.nnzb * p.b * p.b * sizeof(float) : 0;
    d.bias_bytes = (size_t)d.bchunks * p.N * sizeof(float);
    d.partial_off = 0;
    d.bias_off = al(d.partial_bytes);
    d.total = d.bias_off + al(d.bias_bytes);
    return d;
}

int32_t launched(const char *what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(BSR_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
    return BSR_OK;
}

template <int BS, int G, bool TRANS>
void launch_gg(const bsr_pattern &p, const FwdArgs &a, hipStream_t st, int nmtiles) {
    const DeviceMeta &d = p.dev;
    const GroupSchedule &s = TRANS ? p.bwd : p.fwd;
    const dim3 grid((unsigned)((int64_t)s.ngroups * nmtiles));
    hipLaunchKernelGGL((k_group_gemm<BS, G, TRANS>), grid, dim3(kThreads), 0, st, a.act, a.in_ld, a.M, a.V, a.bias,
                       a.out, a.out_ld, TRANS ? d.t_order : d.f_order, TRANS ? d.t_step_ptr : d.f_step_ptr,
                       TRANS ? d.t_out : d.f_out, TRANS ? d.t_step_in : d.f_step_in,
                       TRANS ? d.t_step_blk : d.f_step_blk, nmtiles);
}

}  // namespace

int32_t launch_group_gemm(const bsr_pattern &p, bool transposed, const FwdArgs &a, void *stream) {
    const hipStream_t st = (hipStream_t)stream;
    const int64_t nmt = (a.M + kTileM - 1) / kTileM;
    const GroupSchedule &s = transposed ? p.bwd : p.fwd;
    if (nmt * s.ngroups > (int64_t)INT32_MAX) return fail(BSR_ERR_INVALID_ARG, "problem too large for one launch");
    const int nmtiles = (int)nmt;
    if (p.b == 32) {
        if (transposed) launch_gg<32, kGroupFor32, true>(p, a, st, nmtiles);
        else launch_gg<32, kGroupFor32, false>(p, a, st, nmtiles);
    } else {
        if (transposed) launch_gg<64, kGroupFor64, true>(p, a, st, nmtiles);
        else launch_gg<64, kGroupFor64, false>(p, a, st, nmtiles);
    }
    return launched(transposed ? "bwd_input launch" : "fwd launch");
}

int32_t launch_small_m_fwd(const bsr_pattern &p, const FwdArgs &a, void *stream) {
    const hipStream_t st = (hipStream_t)stream;
    const DeviceMeta &d = p.dev;
    const dim3 grid((unsigned)(p.R * (p.b / 16)));
    if (p.b == 32)
        hipLaunchKernelGGL((k_small_m<32>), grid, dim3(64), 0, st, a.act, p.K, (int)a.M, a.V, a.bias, a.out, p.N,
                           d.row_ptr, d.col_idx, d.rows_by_nnz);
    else
        hipLaunchKernelGGL((k_small_m<64>), grid, dim3(64), 0, st, a.act, p.K, (int)a.M, a.V, a.bias, a.out, p.N,
                           d.row_ptr, d.col_idx, d.rows_by_nnz);
    return launched("fwd small-M launch");
}

size_t dw_workspace_bytes(const bsr_pattern &p, int64_t M) { return M > 0 ? plan_dw(p, M).total : 0; }

int32_t launch_dw(const bsr_pattern &p, const DwArgs &a, void *stream) {
    const hipStream_t st = (hipStream_t)stream;
    const DeviceMeta &d = p.dev;
    const size_t nval = (size_t)p.nnzb * p.b * p.b;
    if (a.M == 0) {
        if (nval) hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)((nval + kThreads - 1) / kThreads)), dim3(kThreads), 0, st,
                                     a.dV, nval);
        if (a.dbias)
            hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)((p.N + kThreads - 1) / kThreads)), dim3(kThreads), 0, st,
                               a.dbias, (size_t)p.N);
        return launched("bwd_weight zero fill");
    }
    const DwPlan pl = plan_dw(p, a.M);
    char *ws = static_cast<char *>(a.ws);
    float *partial = pl.nchunks > 1 ? reinterpret_cast<float *>(ws + pl.partial_off) : nullptr;
    if (p.nnzb > 0) {
        const dim3 grid((unsigned)((int64_t)p.nnzb * pl.nchunks));
        if (p.b == 32)
            hipLaunchKernelGGL((k_dw<32>), grid, dim3(kThreads), 0, st, a.dY, p.N, a.X, p.K, a.M, d.blk_row, d.col_idx,
                               pl.mchunk, pl.nchunks, p.nnzb, partial, a.dV);
        else
            hipLaunchKernelGGL((k_dw<64>), grid, dim3(kThreads), 0, st, a.dY, p.N, a.X, p.K, a.M, d.blk_row, d.col_idx,
                               pl.mchunk, pl.nchunks, p.nnzb, partial, a.dV);
        if (pl.nchunks > 1)
            hipLaunchKernelGGL(k_dw_reduce, dim3((unsigned)((nval + kThreads - 1) / kThreads)), dim3(kThreads), 0, st,
                               partial, pl.nchunks, nval, a.dV);
    }
    if (a.dbias) {
        float *bp = reinterpret_cast<float *>(ws + pl.bias_off);
        hipLaunchKernelGGL(k_colsum_partial, dim3((unsigned)((p.N + kThreads - 1) / kThreads), (unsigned)pl.bchunks),
                           dim3(kThreads), 0, st, a.dY, p.N, a.M, pl.brows, bp);
        hipLaunchKernelGGL(k_colsum_final, dim3((unsigned)((p.N + kThreads - 1) / kThreads)), dim3(kThreads), 0, st, bp,
                           pl.bchunks, p.N, a.dbias);
    }
    return launched("bwd_weight launch");
}

}  // namespace bsr
