// bsr_fp8.hip -- fp8 (OCP E4M3) block values with one power-of-two scale per kept block, and the
// forward for few activation rows that streams them.
//
// For memory-bound layers the pages suggest loading the weights in a compact form and expanding
// them on the GPU before a dense product (Lecture 11 summary, 48:12 "Load and Sparse Expand"), and
// combining sparsity with quantization (same summary, 30:31; pytorch/ao sparsity README: sparsity
// composes with the quantization workflows). At few rows the forward reads almost nothing but the
// block values, so one byte per value instead of two halves the bytes the layer moves.
//
// Format. A kept block i stores b x b E4M3 codes (1 sign bit, 4 exponent bits with bias 7,
// 3 mantissa bits; exponent field 0 holds the subnormals m * 2^-9; largest finite 448) in the same
// order as its bf16 values, and an exponent se[i]: the value of an element is code * 2^se[i].
// se[i] is the smallest integer >= -126 with amax_i <= 448 * 2^se[i] (0 for an all-zero block), so
// no code overflows. Quantisation rounds v / 2^se[i] (exact) to the nearest code, ties to the even
// code; the sign is kept.
//
// The forward expands each code pair with one gfx950 scaled conversion (fp8 -> bf16 times
// 2^se[i], exact for every code at the scales used) and multiplies on the 16x16x32 bf16 matrix
// cores, with the same work split as the bf16 forward for few rows: a work-group takes two
// 16-row slices of one block row's output, rows heaviest first; its waves take the row's blocks a
// few at a time, requesting every load of a pass before the first product; the waves' partial
// sums are added in LDS in wave order.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <string>

#include "bsr_fp8_internal.hpp"

namespace bsr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRawBuffer = 0x00020000;   // raw 32-bit buffer, gfx9 layout

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kRawBuffer);
}

__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

// Eight E4M3 codes (k ascending in the bytes of d0, then d1) -> eight bf16 values code * scale.
__device__ __forceinline__ bf16x8 expand8(uint32_t d0, uint32_t d1, float scale) {
    const u32x4 w = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, scale, false)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, scale, true)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, scale, false)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, scale, true))};
    return __builtin_bit_cast(bf16x8, w);
}

__device__ __forceinline__ uint16_t to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ float from_bf16(uint32_t h) { return __uint_as_float(h << 16); }

// Nearest E4M3 code of x (|x| <= 448, exact in fp32), ties to the even code, sign kept.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
    const uint32_t bits = __float_as_uint(x);
    const uint32_t s = (bits >> 24) & 0x80u;
    const float a = fabsf(x);
    if (a < 0.015625f) {                               // below 2^-6: subnormal grid of step 2^-9
        const uint32_t k = (uint32_t)rintf(a * 512.0f);   // 0 .. 8, round to nearest even
        return s | (k >= 8u ? 0x08u : k);
    }
    const uint32_t ab = __float_as_uint(a);
    int E = (int)(ab >> 23) - 127;                     // -6 .. 8
    uint32_t m = (ab >> 20) & 7u;
    const uint32_t rest = ab & 0xFFFFFu, half = 0x80000u;
    if (rest > half || (rest == half && (m & 1u))) ++m;
    if (m == 8u) {
        m = 0u;
        ++E;
    }
    return s | ((uint32_t)(E + 7) << 3) | m;
}

// Scale exponent of a block from the bits of its largest magnitude (a finite bf16 pattern with the
// sign cleared): the smallest e >= -126 with amax <= 448 * 2^e, 0 for a zero block. With
// amax = (1 + m/128) 2^(E-127): amax <= 448 * 2^e = 1.75 * 2^(e+8) holds for e >= E - 135 when
// m <= 96 (1 + m/128 <= 1.75), else for e >= E - 134.
__device__ __forceinline__ int scale_exponent(uint32_t amax_bits) {
    if (amax_bits == 0u) return 0;
    const int E = (int)(amax_bits >> 7), m = (int)(amax_bits & 0x7Fu);
    if (E == 0) return -126;
    return max(-126, m <= 96 ? E - 135 : E - 134);
}

// One thread per 16 consecutive values of a block of VPB values (b*b for dense blocks, b*b/2 for
// the kept values of 2:4 blocks): TPB = VPB/16 threads per block (32 .. 256); a work-group of 256
// threads covers 256/TPB blocks. The block's largest magnitude is reduced with wave shuffles
// inside groups of min(TPB, 64) lanes, then across the block's waves in LDS.
template <int VPB>
__global__ __launch_bounds__(256) void k_quantize_fp8(const uint16_t *__restrict__ V, int nnzb, uint8_t *__restrict__ V8,
                                                      int32_t *__restrict__ se) {
    constexpr int TPB = VPB / 16, NBW = 256 / TPB, WPB = TPB / 64;
    constexpr int LANES = TPB < 64 ? TPB : 64;
    __shared__ uint32_t wmax[4];
    const int t = threadIdx.x, wave = t >> 6;
    const int i = blockIdx.x * NBW + t / TPB;
    const bool valid = i < nnzb;
    const int64_t off = (int64_t)min(i, nnzb - 1) * VPB + (int64_t)(t % TPB) * 16;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(V + off);
    u32x4 v0 = src[0], v1 = src[1];
    uint32_t w[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    uint32_t amax = 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = max(amax, max(w[j] & 0x7FFFu, (w[j] >> 16) & 0x7FFFu));
#pragma unroll
    for (int o = LANES / 2; o >= 1; o >>= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, o));
    if constexpr (WPB > 1) {
        if ((t & 63) == 0) wmax[wave] = amax;
        __syncthreads();
        const int w0 = wave / WPB * WPB;
#pragma unroll
        for (int k = 0; k < WPB; ++k) amax = max(amax, wmax[w0 + k]);
    }
    const int e = scale_exponent(amax);
    const float inv = pow2f(-e);
    uint32_t out[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t c0 = e4m3_encode(from_bf16(w[2 * j] & 0xFFFFu) * inv);
        const uint32_t c1 = e4m3_encode(from_bf16(w[2 * j] >> 16) * inv);
        const uint32_t c2 = e4m3_encode(from_bf16(w[2 * j + 1] & 0xFFFFu) * inv);
        const uint32_t c3 = e4m3_encode(from_bf16(w[2 * j + 1] >> 16) * inv);
        out[j] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
    }
    if (valid) {
        *reinterpret_cast<u32x4 *>(V8 + off) = u32x4{out[0], out[1], out[2], out[3]};
        if (t % TPB == 0) se[i] = e;
    }
}

// code * 2^se -> bf16, 16 values per thread.
template <int BS>
__global__ __launch_bounds__(256) void k_dequantize_fp8(const uint8_t *__restrict__ V8, const int32_t *__restrict__ se,
                                                        int nnzb, uint16_t *__restrict__ V) {
    constexpr int TPB = BS * BS / 16, NBW = 256 / TPB;
    const int t = threadIdx.x;
    const int i = blockIdx.x * NBW + t / TPB;
    if (i >= nnzb) return;
    const int64_t off = (int64_t)i * BS * BS + (int64_t)(t % TPB) * 16;
    const u32x4 c = *reinterpret_cast<const u32x4 *>(V8 + off);
    const float scale = pow2f(se[i]);
    u32x4 *dst = reinterpret_cast<u32x4 *>(V + off);
    dst[0] = __builtin_bit_cast(u32x4, expand8(c[0], c[1], scale));
    dst[1] = __builtin_bit_cast(u32x4, expand8(c[2], c[3], scale));
}

// ------------------------------------------------------------------------------------------
// Forward, 16 activation rows per grid row y (rows m0 = 16 y .. m0 + 15; past M read as zero):
//   slice s:  A[p][k] = V8[i][s*16 + p][k'] * 2^se[i]   B[k][m] = X[m0 + m][c*BS + k']
// where k' permutes the block's columns so that each lane's codes are one contiguous 8-byte
// (BS = 32) or 16-byte (BS = 64) load: lane group g = lane / 16 owns columns 8 KC g .. 8 KC g +
// 8 KC - 1, and 32-deep chunk kc takes the kc-th 8 of them. A and B use the same permutation, so
// the products are those of the plain definition. Lane l ends up with output columns
// 4 (l / 16) .. + 3 of the slice for activation row l % 16.
// ------------------------------------------------------------------------------------------
template <int BS, int NW, int U, int PSW>
__global__ __launch_bounds__(NW * 64) void k_fwd_fp8(const uint16_t *__restrict__ X, int K, int M,
                                                     const uint8_t *__restrict__ V8, const int32_t *__restrict__ se,
                                                     const uint16_t *__restrict__ bias, uint16_t *__restrict__ Y, int N,
                                                     const int32_t *__restrict__ col_idx,
                                                     const int32_t *__restrict__ rows) {
    constexpr int PS = PSW;
    constexpr int KC = BS / 32;
    constexpr int PARTS = BS / 16 / PSW;
    __shared__ f32x4 red[NW][PS][64];

    const int4 e = reinterpret_cast<const int4 *>(rows)[blockIdx.x / PARTS];
    const int r = e.x, i1 = e.z, s0 = (int)(blockIdx.x % PARTS) * PSW;
    const int m0 = blockIdx.y * 16, Mc = min(16, M - m0);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int l16 = lane & 15, lq = lane >> 4;
    const __amdgpu_buffer_rsrc_t rx = rsrc(X + (int64_t)m0 * K, (uint32_t)Mc * K * 2);
    const uint32_t xoff = (uint32_t)(l16 * K + lq * 8 * KC) * 2;
    const uint32_t xend = (uint32_t)Mc * K * 2;   // past this chunk's activations: reads zeros
    const uint32_t voff = (uint32_t)((s0 * 16 + l16) * BS + lq * 8 * KC);

    f32x4 acc[PS];
#pragma unroll
    for (int s = 0; s < PS; ++s) acc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int i0 = e.y; i0 < i1; i0 += NW * U) {
        const int ib = i0 + wave * U;
        u32x4 code[U][PS];     // KC = 2: 16 codes; KC = 1: 8 codes in .x, .y
        bf16x8 b[U][KC];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int iu = ib + u;
            const __amdgpu_buffer_rsrc_t rv = rsrc(V8 + (size_t)min(iu, i1 - 1) * BS * BS, iu < i1 ? BS * BS : 0);
#pragma unroll
            for (int s = 0; s < PS; ++s) {
                if (KC == 2) {
                    code[u][s] = __builtin_amdgcn_raw_buffer_load_b128(rv, voff + s * 16 * BS, 0, 0);
                } else {
                    const u32x2 c2 = __builtin_amdgcn_raw_buffer_load_b64(rv, voff + s * 16 * BS, 0, 0);
                    code[u][s] = u32x4{c2[0], c2[1], 0u, 0u};
                }
            }
        }
        int col[U], ex[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            col[u] = col_idx[min(ib + u, i1 - 1)];
            ex[u] = se[min(ib + u, i1 - 1)];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // blocks past the row's end read zeros for both operands
            const uint32_t xo = ib + u < i1 ? xoff : xend;
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
                b[u][kc] = __builtin_bit_cast(
                    bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rx, xo + kc * 16, (uint32_t)col[u] * BS * 2, 0));
        }
        __builtin_amdgcn_sched_barrier(0);   // keep the products after every load
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float scale = pow2f(ex[u]);
#pragma unroll
            for (int s = 0; s < PS; ++s)
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) {
                    const bf16x8 a = expand8(code[u][s][2 * kc], code[u][s][2 * kc + 1], scale);
                    acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[u][kc], acc[s], 0, 0, 0);
                }
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

// Rows (block rows of zero blocks) with no kept block still need Y = bias (or 0): the row list
// holds every block row, so each work-group writes its slices even when its loop is empty.

int32_t launched(const char *what) {
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return fail(BSR_ERR_HIP, std::string(what) + ": " + hipGetErrorString(err));
    return BSR_OK;
}

template <int BS>
int blocks_per_wg() {
    return 256 / (BS * BS / 16);
}

}  // namespace

template <int VPB>
void launch_quantize_vpb(int nnzb, const uint16_t *V, uint8_t *V8, int32_t *se, hipStream_t st) {
    constexpr int NBW = 256 / (VPB / 16);
    hipLaunchKernelGGL((k_quantize_fp8<VPB>), dim3((unsigned)((nnzb + NBW - 1) / NBW)), dim3(256), 0, st, V, nnzb, V8,
                       se);
}

int32_t launch_quantize_fp8(const bsr_pattern &p, const uint16_t *V, uint8_t *V8, int32_t *se, void *stream,
                            bool kept24) {
    if (p.nnzb == 0) return BSR_OK;
    const hipStream_t st = (hipStream_t)stream;
    if (p.b == 32) {
        if (kept24) launch_quantize_vpb<32 * 16>(p.nnzb, V, V8, se, st);
        else launch_quantize_vpb<32 * 32>(p.nnzb, V, V8, se, st);
    } else {
        if (kept24) launch_quantize_vpb<64 * 32>(p.nnzb, V, V8, se, st);
        else launch_quantize_vpb<64 * 64>(p.nnzb, V, V8, se, st);
    }
    return launched("quantize_fp8 launch");
}

int32_t launch_dequantize_fp8(const bsr_pattern &p, const uint8_t *V8, const int32_t *se, uint16_t *V, void *stream) {
    if (p.nnzb == 0) return BSR_OK;
    const hipStream_t st = (hipStream_t)stream;
    if (p.b == 32) {
        const dim3 grid((unsigned)((p.nnzb + blocks_per_wg<32>() - 1) / blocks_per_wg<32>()));
        hipLaunchKernelGGL((k_dequantize_fp8<32>), grid, dim3(256), 0, st, V8, se, p.nnzb, V);
    } else {
        const dim3 grid((unsigned)((p.nnzb + blocks_per_wg<64>() - 1) / blocks_per_wg<64>()));
        hipLaunchKernelGGL((k_dequantize_fp8<64>), grid, dim3(256), 0, st, V8, se, p.nnzb, V);
    }
    return launched("dequantize_fp8 launch");
}

template <int BS, int NW, int U, int PSW>
void launch_fwd_fp8_cfg(const bsr_pattern &p, const uint16_t *X, int64_t M, const uint8_t *V8, const int32_t *se,
                        const uint16_t *bias, uint16_t *Y, hipStream_t st) {
    const dim3 grid((unsigned)(p.R * (BS / 16 / PSW)), (unsigned)((M + 15) / 16));
    hipLaunchKernelGGL((k_fwd_fp8<BS, NW, U, PSW>), grid, dim3(NW * 64), 0, st, X, p.K, (int)M, V8, se, bias, Y, p.N,
                       p.dev.col_idx, p.dev.small_m_rows);
}

int32_t launch_fwd_fp8(const bsr_pattern &p, const uint16_t *X, int64_t M, const uint8_t *V8, const int32_t *se,
                       const uint16_t *bias, uint16_t *Y, void *stream) {
    const hipStream_t st = (hipStream_t)stream;
    // b = 32: 8 waves x 8 blocks in flight, both slices of a block per work-group. b = 64: waves,
    // blocks in flight per wave and 16-row slices per work-group (of 4) by configuration.
    if (p.b == 32) {
        launch_fwd_fp8_cfg<32, 8, 8, 2>(p, X, M, V8, se, bias, Y, st);
        return launched("fwd_fp8 launch");
    }
    int cfg = 0;
    if (const char *f = std::getenv("BSR_FP8_CONFIG")) cfg = std::atoi(f);   // tuning knob: 0 .. 7
    switch (cfg) {
        case 1: launch_fwd_fp8_cfg<64, 8, 4, 1>(p, X, M, V8, se, bias, Y, st); break;
        case 2: launch_fwd_fp8_cfg<64, 8, 2, 1>(p, X, M, V8, se, bias, Y, st); break;
        case 3: launch_fwd_fp8_cfg<64, 8, 8, 2>(p, X, M, V8, se, bias, Y, st); break;
        case 4: launch_fwd_fp8_cfg<64, 4, 4, 1>(p, X, M, V8, se, bias, Y, st); break;
        case 5: launch_fwd_fp8_cfg<64, 16, 2, 1>(p, X, M, V8, se, bias, Y, st); break;
        case 6: launch_fwd_fp8_cfg<64, 16, 4, 2>(p, X, M, V8, se, bias, Y, st); break;
        case 7: launch_fwd_fp8_cfg<64, 4, 8, 1>(p, X, M, V8, se, bias, Y, st); break;
        default: launch_fwd_fp8_cfg<64, 8, 4, 2>(p, X, M, V8, se, bias, Y, st); break;
    }
    return launched("fwd_fp8 launch");
}

}  // namespace bsr
