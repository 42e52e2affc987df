// bsr_sparse24.hip -- 2:4 sparsity inside each kept block, and the forward for few activation rows
// on the gfx950 sparse matrix cores.
//
// The pattern of 50% sparsity inside blocks is on the block-sparse layer's roadmap
// (pytorch_block_sparse summary page, "Future Development Roadmap"); 2:4 means two of every four
// consecutive elements are zero, pruned by norm over 1 x 4 groups, and is stored as a half-size
// compressed matrix plus 2-bit indices (pytorch/ao sparsity README, workflow example and Table 4.1).
//
// Format. In every row p of kept block i, each group of 4 consecutive columns (the input dimension,
// which the forward sums over) keeps its two elements of largest magnitude, ties to the lower
// position, in ascending position order:
//   Vc[i][p][2h + t]    the t-th kept value of group h                    (bf16, [nnzb][b][b/2])
//   meta[i][p][h / 4]   group h at bits 4 (h % 4): first position in the low 2 bits, second in the
//                       next 2 (uint16, [nnzb][b][b/16])
// which is the index layout v_smfmac_f32_16x16x64_bf16 takes for its sparse operand.
//
// Forward for few rows: the same work split as the bf16 one (two 16-row output slices of one block
// row per work-group, rows heaviest first, every load of a pass before the products, partial sums
// added in LDS in wave order). One sparse MFMA contracts 64 columns: for b = 64 one block, for
// b = 32 two consecutive kept blocks of the row (lane groups 0-1 take the first, 2-3 the second).
// Operand layout of the instruction (measured with a probe on the box: every one of eight random
// trials matched bit for bit):
//   sparse A (16 x 64, 8 kept values per lane): lane l holds row l % 16, dense columns
//       16 (l / 16) .. + 15 (four groups), with 2 index bits per kept value;
//   dense B (64 x 16, 16 values per lane): lane l holds column l % 16, rows 8 (l / 16) .. + 7 in
//       its first 8 values and 32 + 8 (l / 16) .. + 7 in the last 8;
//   D as for the dense 16 x 16 instructions: lane l holds column l % 16, rows 4 (l / 16) .. + 3.
// With A = a 16-row slice of the compressed block and B = activation rows, D holds Y^T.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "bsr_sparse24_internal.hpp"

namespace bsr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x8 __attribute__((ext_vector_type(8)));

constexpr int kRawBuffer = 0x00020000;    // raw 32-bit buffer, gfx9 layout
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;   // a buffer offset past every buffer here: reads zeros

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kRawBuffer);
}

// Eight E4M3 codes (ascending in the bytes of d0, then d1) -> eight bf16 values code * scale (the
// gfx950 scaled conversion uses only the exponent of the scale, a power of two here).
__device__ __forceinline__ bf16x8 expand8(uint32_t d0, uint32_t d1, float scale) {
    const u32x4 w = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, scale, false)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, scale, true)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, scale, false)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, scale, true))};
    return __builtin_bit_cast(bf16x8, w);
}

__device__ __forceinline__ uint16_t to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ float from_bf16(uint32_t h) { return __uint_as_float(h << 16); }

// One thread per 16 columns (4 groups) of one block row.
template <int BS>
__global__ __launch_bounds__(256) void k_compress_24(const uint16_t *__restrict__ V, int64_t segments,
                                                     uint16_t *__restrict__ Vc, uint16_t *__restrict__ meta) {
    const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;   // segment: 16 columns of one block row
    if (s >= segments) return;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(V + s * 16);
    const u32x4 w0 = src[0], w1 = src[1];
    const uint32_t w[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
    uint32_t out[4];
    uint32_t bits = 0;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const uint32_t v[4] = {w[2 * h] & 0xFFFFu, w[2 * h] >> 16, w[2 * h + 1] & 0xFFFFu, w[2 * h + 1] >> 16};
        // magnitudes compare as the integers of the bits with the sign cleared (finite values)
        int first = 0;
#pragma unroll
        for (int k = 1; k < 4; ++k)
            if ((v[k] & 0x7FFFu) > (v[first] & 0x7FFFu)) first = k;
        int second = first == 0 ? 1 : 0;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (k != first && k != second && (v[k] & 0x7FFFu) > (v[second] & 0x7FFFu)) second = k;
        // `second` starts at the lowest position other than `first`; later positions replace it only
        // when strictly larger, so among equals the lower position is kept
        const int lo = min(first, second), hi = max(first, second);
        out[h] = v[lo] | (v[hi] << 16);
        bits |= (uint32_t)(lo | (hi << 2)) << (4 * h);
    }
    *reinterpret_cast<u32x4 *>(Vc + s * 8) = u32x4{out[0], out[1], out[2], out[3]};
    meta[s] = (uint16_t)bits;
}

template <int BS>
__global__ __launch_bounds__(256) void k_decompress_24(const uint16_t *__restrict__ Vc,
                                                       const uint16_t *__restrict__ meta, int64_t segments,
                                                       uint16_t *__restrict__ V) {
    const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (s >= segments) return;
    const u32x4 c = *reinterpret_cast<const u32x4 *>(Vc + s * 8);
    const uint32_t bits = meta[s];
    uint32_t d[8];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const uint32_t nib = (bits >> (4 * h)) & 15u, lo = nib & 3u, hi = nib >> 2;
        uint16_t g[4] = {0, 0, 0, 0};
        g[lo] = (uint16_t)(c[h] & 0xFFFFu);
        g[hi] = (uint16_t)(c[h] >> 16);
        d[2 * h] = g[0] | ((uint32_t)g[1] << 16);
        d[2 * h + 1] = g[2] | ((uint32_t)g[3] << 16);
    }
    u32x4 *dst = reinterpret_cast<u32x4 *>(V + s * 16);
    dst[0] = u32x4{d[0], d[1], d[2], d[3]};
    dst[1] = u32x4{d[4], d[5], d[6], d[7]};
}

// Forward: grid (R * BS / 16 / PSW, ceil(M / 16)). A unit is what one sparse MFMA contracts:
// 64 columns = UB = 64 / BS consecutive kept blocks of the row.
// F8: the kept values are E4M3 codes with one power-of-two scale per block (se), expanded to bf16
// by the gfx950 scaled conversion (two codes per instruction) before the product.
template <int BS, int NW, int U, int PSW, bool F8>
__global__ __launch_bounds__(NW * 64) void k_fwd_24(const uint16_t *__restrict__ X, int K, int M,
                                                    const void *__restrict__ Vc, const int32_t *__restrict__ se,
                                                    const uint16_t *__restrict__ meta,
                                                    uint32_t vc_bytes, uint32_t meta_bytes,
                                                    const uint16_t *__restrict__ bias, uint16_t *__restrict__ Y, int N,
                                                    const int32_t *__restrict__ col_idx,
                                                    const int32_t *__restrict__ rows) {
    constexpr int PS = PSW;
    constexpr int UB = 64 / BS;              // kept blocks per unit
    constexpr int PARTS = BS / 16 / PSW;
    constexpr int CPR = BS / 16;             // 16-column chunks per block row
    __shared__ f32x4 red[NW][PS][64];

    const int4 e = reinterpret_cast<const int4 *>(rows)[blockIdx.x / PARTS];
    const int r = e.x, i1 = e.z, s0 = (int)(blockIdx.x % PARTS) * PSW;
    const int m0 = blockIdx.y * 16, Mc = min(16, M - m0);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int l16 = lane & 15, lq = lane >> 4;
    const __amdgpu_buffer_rsrc_t rx = rsrc(X + (int64_t)m0 * K, (uint32_t)Mc * K * 2);
    const __amdgpu_buffer_rsrc_t rv = rsrc(Vc, vc_bytes);
    const __amdgpu_buffer_rsrc_t rm = rsrc(meta, meta_bytes);
    const uint32_t xend = (uint32_t)Mc * K * 2;   // past this chunk's activations: reads zeros
    // sparse operand: this lane's block of the unit and its 16-column chunk inside the block
    const int a_blk = UB == 1 ? 0 : lq >> 1, a_chunk = UB == 1 ? lq : lq & 1;
    // dense operand: the block of each 8-column half, and the half's first column inside it
    const int b_blk1 = UB == 1 ? 0 : 1;
    const int b_col0 = 8 * lq, b_col1 = UB == 1 ? 32 + 8 * lq : 8 * lq;

    f32x4 acc[PS];
#pragma unroll
    for (int s = 0; s < PS; ++s) acc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int i0 = e.y; i0 < i1; i0 += NW * U * UB) {
        const int ib = i0 + wave * U * UB;
        bf16x8 a[U][PS];
        u32x2 code[U][PS];
        int idx[U][PS];
        int ex[U];
        bf16x16 bx[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int ia = ib + u * UB + a_blk;
#pragma unroll
            for (int s = 0; s < PS; ++s) {
                const int p = (s0 + s) * 16 + l16;
                const uint32_t row = (uint32_t)ia * BS + p;
                constexpr uint32_t VB = F8 ? 1 : 2;   // bytes per kept value
                const uint32_t vo = ia < i1 ? (row * (BS / 2) + a_chunk * 8) * VB : kOutOfRange;
                const uint32_t mo = ia < i1 ? (row * CPR + a_chunk) * 2 : kOutOfRange;
                if constexpr (F8) {
                    const u32x2 c = __builtin_amdgcn_raw_buffer_load_b64(rv, vo, 0, 0);
                    code[u][s] = c;
                } else {
                    a[u][s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rv, vo, 0, 0));
                }
                idx[u][s] = (int)(uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rm, mo, 0, 0);
            }
        }
        if constexpr (F8) {
#pragma unroll
            for (int u = 0; u < U; ++u) ex[u] = se[min(ib + u * UB + a_blk, i1 - 1)];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j0 = ib + u * UB, j1 = j0 + b_blk1;
            const int c0 = col_idx[min(j0, i1 - 1)], c1 = col_idx[min(j1, i1 - 1)];
            // blocks past the row's end read zeros for both operands
            const uint32_t x0 = j0 < i1 ? (uint32_t)(l16 * K + c0 * BS + b_col0) * 2 : xend;
            const uint32_t x1 = j1 < i1 ? (uint32_t)(l16 * K + c1 * BS + b_col1) * 2 : xend;
            const u32x4 h0 = __builtin_amdgcn_raw_buffer_load_b128(rx, x0, 0, 0);
            const u32x4 h1 = __builtin_amdgcn_raw_buffer_load_b128(rx, x1, 0, 0);
            bx[u] = __builtin_bit_cast(bf16x16, u32x8{h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]});
        }
        __builtin_amdgcn_sched_barrier(0);   // keep the products after every load
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if constexpr (F8) {
                const float scale = __uint_as_float((uint32_t)(ex[u] + 127) << 23);
#pragma unroll
                for (int s = 0; s < PS; ++s) a[u][s] = expand8(code[u][s][0], code[u][s][1], scale);
            }
#pragma unroll
            for (int s = 0; s < PS; ++s)
                acc[s] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(a[u][s], bx[u], acc[s], idx[u][s], 0, 0);
        }
    }
#pragma unroll
    for (int s = 0; s < PS; ++s) red[wave][s][lane] = acc[s];
    __syncthreads();
    if (wave < PS) {
        f32x4 v = red[0][wave][lane];
#pragma unroll
        for (int w = 1; w < NW; ++w) v += red[w][wave][lane];
        if (l16 < Mc) {
            const int n = r * BS + (s0 + wave) * 16 + lq * 4;
            if (bias) {
                const uint2 bb = *reinterpret_cast<const uint2 *>(bias + n);
                v[0] += from_bf16(bb.x & 0xffffu);
                v[1] += from_bf16(bb.x >> 16);
                v[2] += from_bf16(bb.y & 0xffffu);
                v[3] += from_bf16(bb.y >> 16);
            }
            const uint32_t lo = (uint32_t)to_bf16(v[0]) | ((uint32_t)to_bf16(v[1]) << 16);
            const uint32_t hi = (uint32_t)to_bf16(v[2]) | ((uint32_t)to_bf16(v[3]) << 16);
            *reinterpret_cast<uint2 *>(Y + (int64_t)(m0 + l16) * N + n) = make_uint2(lo, hi);
        }
    }
}

// 2:4 image of a block for the large-M forward: the size of a bf16 block ([b][b] 16-bit units,
// 2b bytes per row), row n = the row's b/2 kept values (b bytes), then its b/16 index words
// (b/8 bytes), then zeros. One thread per block row.
template <int BS>
__global__ __launch_bounds__(256) void k_pack_24(const uint16_t *__restrict__ Vc, const uint16_t *__restrict__ meta,
                                                 int64_t nrows, uint16_t *__restrict__ img) {
    const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (row >= nrows) return;
    constexpr int VC = BS / 16;        // 16-byte chunks of kept values per row (2 or 4)
    const u32x4 *src = reinterpret_cast<const u32x4 *>(Vc + row * (BS / 2));
    u32x4 *dst = reinterpret_cast<u32x4 *>(img + row * BS);
#pragma unroll
    for (int c = 0; c < VC; ++c) dst[c] = src[c];
    const uint16_t *m = meta + row * (BS / 16);
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < BS / 16; ++k) w[k / 2] |= (uint32_t)m[k] << (16 * (k % 2));
    dst[VC] = u32x4{w[0], w[1], w[2], w[3]};
#pragma unroll
    for (int c = VC + 1; c < 2 * BS / 16; ++c) dst[c] = u32x4{0u, 0u, 0u, 0u};
}

int32_t launched(const char *what) {
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return fail(BSR_ERR_HIP, std::string(what) + ": " + hipGetErrorString(err));
    return BSR_OK;
}

}  // namespace

int32_t launch_compress_24(const bsr_pattern &p, const uint16_t *V, uint16_t *Vc, uint16_t *meta, void *stream) {
    const int64_t segments = (int64_t)p.nnzb * p.b * (p.b / 16);
    if (segments == 0) return BSR_OK;
    const dim3 grid((unsigned)((segments + 255) / 256));
    const hipStream_t st = (hipStream_t)stream;
    if (p.b == 32)
        hipLaunchKernelGGL((k_compress_24<32>), grid, dim3(256), 0, st, V, segments, Vc, meta);
    else
        hipLaunchKernelGGL((k_compress_24<64>), grid, dim3(256), 0, st, V, segments, Vc, meta);
    return launched("compress_24 launch");
}

int32_t launch_decompress_24(const bsr_pattern &p, const uint16_t *Vc, const uint16_t *meta, uint16_t *V,
                             void *stream) {
    const int64_t segments = (int64_t)p.nnzb * p.b * (p.b / 16);
    if (segments == 0) return BSR_OK;
    const dim3 grid((unsigned)((segments + 255) / 256));
    const hipStream_t st = (hipStream_t)stream;
    if (p.b == 32)
        hipLaunchKernelGGL((k_decompress_24<32>), grid, dim3(256), 0, st, Vc, meta, segments, V);
    else
        hipLaunchKernelGGL((k_decompress_24<64>), grid, dim3(256), 0, st, Vc, meta, segments, V);
    return launched("decompress_24 launch");
}

int32_t launch_pack_24(const bsr_pattern &p, const uint16_t *Vc, const uint16_t *meta, uint16_t *img, void *stream) {
    const int64_t nrows = (int64_t)p.nnzb * p.b;
    if (nrows == 0) return BSR_OK;
    const dim3 grid((unsigned)((nrows + 255) / 256));
    const hipStream_t st = (hipStream_t)stream;
    if (p.b == 32)
        hipLaunchKernelGGL((k_pack_24<32>), grid, dim3(256), 0, st, Vc, meta, nrows, img);
    else
        hipLaunchKernelGGL((k_pack_24<64>), grid, dim3(256), 0, st, Vc, meta, nrows, img);
    return launched("pack_24 launch");
}

template <bool F8>
int32_t launch_fwd_24_impl(const bsr_pattern &p, const uint16_t *X, int64_t M, const void *Vc, const int32_t *se,
                           const uint16_t *meta, const uint16_t *bias, uint16_t *Y, hipStream_t st) {
    const uint32_t vc_bytes = (uint32_t)((size_t)p.nnzb * p.b * (p.b / 2) * (F8 ? 1 : 2));
    const uint32_t meta_bytes = (uint32_t)((size_t)p.nnzb * p.b * (p.b / 16) * 2);
    const unsigned chunks = (unsigned)((M + 15) / 16);
    // 8 waves x 4 units (4 blocks for b = 64, 8 for b = 32) in flight, two of the b/16 slices per
    // work-group
    if (p.b == 32) {
        const dim3 grid((unsigned)(p.R * (2 / 2)), chunks);
        hipLaunchKernelGGL((k_fwd_24<32, 8, 4, 2, F8>), grid, dim3(512), 0, st, X, p.K, (int)M, Vc, se, meta, vc_bytes,
                           meta_bytes, bias, Y, p.N, p.dev.col_idx, p.dev.small_m_rows);
    } else {
        const dim3 grid((unsigned)(p.R * (4 / 2)), chunks);
        hipLaunchKernelGGL((k_fwd_24<64, 8, 4, 2, F8>), grid, dim3(512), 0, st, X, p.K, (int)M, Vc, se, meta, vc_bytes,
                           meta_bytes, bias, Y, p.N, p.dev.col_idx, p.dev.small_m_rows);
    }
    return launched(F8 ? "fwd_fp8_24 launch" : "fwd_24 launch");
}

int32_t launch_fwd_24(const bsr_pattern &p, const uint16_t *X, int64_t M, const uint16_t *Vc, const uint16_t *meta,
                      const uint16_t *bias, uint16_t *Y, void *stream) {
    return launch_fwd_24_impl<false>(p, X, M, Vc, nullptr, meta, bias, Y, (hipStream_t)stream);
}

int32_t launch_fwd_fp8_24(const bsr_pattern &p, const uint16_t *X, int64_t M, const uint8_t *Vc8, const int32_t *se,
                          const uint16_t *meta, const uint16_t *bias, uint16_t *Y, void *stream) {
    return launch_fwd_24_impl<true>(p, X, M, Vc8, se, meta, bias, Y, (hipStream_t)stream);
}

}  // namespace bsr
