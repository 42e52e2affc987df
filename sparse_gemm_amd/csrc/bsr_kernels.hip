// bsr_kernels.hip -- gfx950 (CDNA4) kernels of the block-sparse linear layer.
//
// Every kept b x b block is a real dense contraction, so each one runs on bf16 MFMA with fp32
// accumulation (pytorch_block_sparse summary page, "Technical Foundation": dense matrix-core
// products on the kept blocks, zero blocks skipped). Each output element is rounded once to bf16.
//
// All products use v_mfma_f32_16x16x32_bf16 (wave64). Lane l holds A[l%16][8*(l/16) + t] and
// B[8*(l/16) + t][l%16] for t = 0..7; result item v of lane l is D[4*(l/16) + v][l%16]. Only the
// pairing of A's and B's k positions matters for the sum, so both operands always take the same
// k for the same (lane group, item).
//
// ds_read_b64_tr_b16 (transposing LDS read): in each group of 16 lanes, lane s supplies the
// address of 4 consecutive 16-bit values; lane i = 4u + v receives, as item t, value v of lane
// 4t + u. Pointing lane s at T[k0 + s/4][n0 + 4*(s%4)] of a row-major T[k][n] tile hands lane i
// the values T[k0..k0+3][n0 + i]: a k-run for one n, the MFMA operand layout of a tile that is
// stored n-contiguous.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>

#include "bsr_internal.hpp"

namespace bsr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kCUs = 256;   // compute units of one MI355X
constexpr int kXCDs = 8;    // accelerator complex dies; work-groups go to them round-robin

// Logical index of work-group `bid` such that each XCD's work-groups (bid = x, x + 8, ...) take
// one contiguous run of logical indices, in dispatch order.
__device__ __forceinline__ int xcd_remap(int bid, int nwg) {
    const int xcd = bid % kXCDs, slot = bid / kXCDs;
    const int per = nwg / kXCDs, rem = nwg % kXCDs;
    return xcd * per + min(xcd, rem) + slot;
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Buffer resources: a base address and a size in bytes. A buffer load whose offset lies past the
// size returns zeros and touches no memory, so loads can be issued unconditionally (which keeps
// the compiler's count of loads in flight exact) while rows past the end of a tile or absent
// blocks cost nothing.
constexpr int kBufferFlags = 0x00020000;   // raw 32-bit buffer, gfx9 layout

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kBufferFlags);
}

__device__ __forceinline__ bf16x8 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

__device__ __forceinline__ u32x4 buf_load16u(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}

// Two transposing LDS reads -> one 8-value MFMA operand: T[k0..k0+7][n0 + lane16] of a row-major
// tile T with row pitch `ld` elements.
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

__device__ __forceinline__ f32x4 add_bias4(f32x4 v, const uint16_t *bias) {
    const uint2 bb = *reinterpret_cast<const uint2 *>(bias);
    v[0] += from_bf16(bb.x & 0xffff);
    v[1] += from_bf16(bb.x >> 16);
    v[2] += from_bf16(bb.y & 0xffff);
    v[3] += from_bf16(bb.y >> 16);
    return v;
}

// ------------------------------------------------------------------------------------------
// Group GEMM: forward (TRANS = false) and input gradient (TRANS = true).
//
// A work-group owns G output blocks (block rows of W for the forward, block columns for the
// input gradient) and BM = NW * WM activation rows; wave w owns rows [w*WM, (w+1)*WM) of them for
// all G blocks, so every wave does the same work whatever blocks are present. A step takes one
// input block of the activations (block column c of X, or block row r of dY) and the value blocks
// of the members that have a kept block there:
//   out tile^T [n][m] += A[n][k] . B[k][m],   B[k][m] = act[m][in*BS + k]
//   forward:    A[n][k] = V[i][n][k]   (natural layout, 16-byte LDS reads)
//   input grad: A[n][k] = V[i][k][n]   (transposed, ds_read_b64_tr_b16 of the natural layout)
// so each lane ends up with 4 consecutive output columns of one activation row.
// Pipelining: at step s the activation fragments and the value blocks of step s + P are loaded
// into registers (rings of P slots) while step s computes; the value blocks of step s + 1, loaded
// P - 1 steps earlier, are then written to the other half of a double-buffered LDS stage. Steps
// come in multiples of P, so the unrolled loop issues the same loads on every trip and the wait
// counts before each use stay exact.
// ------------------------------------------------------------------------------------------
template <int BS, int G, int WM, int NW, int P, bool TRANS>
__global__ __launch_bounds__(NW * 64) void k_group_gemm(
    const uint16_t *__restrict__ act, int in_ld, int M, const uint16_t *__restrict__ V,
    const uint16_t *__restrict__ bias, uint16_t *__restrict__ out, int out_ld, const int32_t *__restrict__ order,
    const int32_t *__restrict__ step_ptr, const int32_t *__restrict__ gout, const int32_t *__restrict__ rec,
    const int32_t *__restrict__ hdr, int nmtiles) {
    constexpr int NT = BS / 16;             // 16-wide output tiles per block
    constexpr int KC = BS / 32;             // 32-deep k chunks per block
    constexpr int MT = WM / 16;             // 16-row activation tiles per wave
    constexpr int BM = WM * NW;
    constexpr int LDW = BS + 8;             // padded LDS pitch of a staged block (elements)
    constexpr int NTH = NW * 64;
    constexpr int CPB = BS * BS / 8;        // 16-byte chunks per block
    constexpr int CPT = G * CPB / NTH;      // chunks per thread per step
    constexpr int RS = rec_stride(G), HS = hdr_stride(G, P);
    static_assert((G * CPB) % NTH == 0 && CPB % 64 == 0, "block staging must divide evenly");
    __shared__ __attribute__((aligned(16))) uint16_t wl[2][G][BS][LDW];

    // Work-groups are dispatched to the 8 XCDs round-robin; give each XCD a contiguous run of
    // logical tiles, ordered activation-tile-major, so that the groups sharing an activation tile
    // run together on one XCD and find it in that XCD's L2.
    const int ngroups = (int)(gridDim.x / nmtiles);
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int g = order[L % ngroups];
    const int mt0 = L / ngroups;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, lq = lane >> 4;
    const int mbase = mt0 * BM + wave * WM;
    const int rlane = min(lane, RS - 1);

    // Activations of this work-group's rows; rows past M read as zeros.
    const int rows = min(BM, M - mt0 * BM);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(act + (int64_t)mt0 * BM * in_ld, (uint32_t)rows * in_ld * 2);
    uint32_t voff[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) voff[mt] = (uint32_t)(((wave * WM + mt * 16 + l16) * in_ld + lq * 8) * 2);

    f32x4 acc[G][NT][MT];
#pragma unroll
    for (int t = 0; t < G; ++t)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[t][nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int s0 = step_ptr[g], s1 = step_ptr[g + 1];
    bf16x8 xr[P][MT][KC];   // activation fragments of the next P steps (ring)
    int rv[P];              // step records of the next P steps (ring; lane k holds word k)
    u32x4 wr[P][CPT];       // value-block chunks of the next P steps (ring)

    auto load_x = [&](bf16x8(&slot)[MT][KC], int in_blk) __attribute__((always_inline)) {
        const uint32_t soff = (uint32_t)in_blk * BS * 2;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) slot[mt][kc] = buf_load16(ra, voff[mt] + kc * 64, soff);
    };
    // value blocks of one step: word `first + t` of record `r` is member t's block (-1 = none)
    auto load_w = [&](u32x4(&slot)[CPT], int r, int first) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int t = (j * NTH + wave * 64) / CPB;   // uniform per wave
            const int w = (tid + j * NTH) % CPB;
            const int blk = __builtin_amdgcn_readlane(r, first + t);
            const __amdgpu_buffer_rsrc_t rw = make_rsrc(V + (size_t)max(blk, 0) * BS * BS, blk >= 0 ? BS * BS * 2 : 0);
            slot[j] = buf_load16u(rw, (uint32_t)w * 16, 0);
        }
    };
    auto store_w = [&](int buf, const u32x4(&slot)[CPT]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int t = (j * NTH + wave * 64) / CPB;
            const int w = (tid + j * NTH) % CPB;
            *reinterpret_cast<u32x4 *>(&wl[buf][t][w / (BS / 8)][(w % (BS / 8)) * 8]) = slot[j];
        }
    };
    auto compute = [&](int buf, const bf16x8(&slot)[MT][KC], int mask) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < G; ++t) {
            if (!((mask >> t) & 1)) continue;   // uniform over the work-group
            bf16x8 a[NT][KC];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) {
                    if constexpr (!TRANS)
                        a[nt][kc] = *reinterpret_cast<const bf16x8 *>(&wl[buf][t][nt * 16 + l16][kc * 32 + lq * 8]);
                    else
                        a[nt][kc] = lds_read_tr8(&wl[buf][t][0][0], LDW, kc * 32 + lq * 8, nt * 16, l16);
                }
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int kc = 0; kc < KC; ++kc) acc[t][nt][mt] = mfma(a[nt][kc], slot[mt][kc], acc[t][nt][mt]);
        }
    };

    if (s0 < s1) {
        const int h = hdr[(size_t)g * HS + min(lane, HS - 1)];
#pragma unroll
        for (int u = 0; u < P; ++u) {
            rv[u] = rec[(size_t)(s0 + u) * RS + rlane];
            load_x(xr[u], __builtin_amdgcn_readlane(h, u));
            load_w(wr[u], h, P + u * G);
        }
        store_w(0, wr[0]);
        __builtin_amdgcn_s_waitcnt(0);   // drain: the loop's wait counts then hold on entry too
        __syncthreads();
        for (int s = s0; s < s1; s += P) {
#pragma unroll
            for (int u = 0; u < P; ++u) {
                const int cs = s + u;
                const int buf = (cs - s0) & 1;
                const int r = rv[u];
                load_w(wr[u], r, 2);                             // value blocks of step cs + P
                compute(buf, xr[u], __builtin_amdgcn_readlane(r, 0));
                load_x(xr[u], __builtin_amdgcn_readlane(r, 1));  // activations of step cs + P
                rv[u] = rec[(size_t)min(cs + P, s1 - 1) * RS + rlane];
                store_w(buf ^ 1, wr[(u + 1) % P]);               // value blocks of step cs + 1
                __syncthreads();
            }
        }
    }

    // Epilogue: item v of lane l is output column nt*16 + 4*(l/16) + v of the block, activation
    // row mt*16 + l%16 of the wave.
#pragma unroll
    for (int t = 0; t < G; ++t) {
        const int o = gout[g * G + t];
        if (o < 0) continue;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = mbase + mt * 16 + l16;
            if (m >= M) continue;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int n = o * BS + nt * 16 + lq * 4;
                f32x4 v = acc[t][nt][mt];
                if (bias) v = add_bias4(v, bias + n);
                store4_bf16(out + (int64_t)m * out_ld + n, v[0], v[1], v[2], v[3]);
            }
        }
    }
}

// ------------------------------------------------------------------------------------------
// Small-M forward (M <= 16): a streaming pass over the block values, the memory-bound regime
// where the kept blocks are loaded once and expanded into dense matrix-core products (GPU MODE
// lecture 11 summary, 48:12, "load and sparse expand"). Work-group = (block row, 16-row slice of
// the block); its 4 waves take the row's kept blocks round-robin, each keeping U blocks of loads
// in flight, and their partial products are summed in LDS in wave order (deterministic).
//   A[p][k] = V[i][slice*16 + p][k]   B[k][m] = X[m][c*BS + k]   (m < 16; rows past M are 0)
// ------------------------------------------------------------------------------------------
template <int BS>
__global__ __launch_bounds__(256) void k_small_m(const uint16_t *__restrict__ X, int K, int M,
                                                 const uint16_t *__restrict__ V, const uint16_t *__restrict__ bias,
                                                 uint16_t *__restrict__ Y, int N, const int32_t *__restrict__ row_ptr,
                                                 const int32_t *__restrict__ col_idx,
                                                 const int32_t *__restrict__ rows_by_nnz) {
    constexpr int PS = BS / 16;   // 16-row slices per block
    constexpr int KC = BS / 32;   // 32-deep k chunks per block
    constexpr int U = 8 / KC;     // blocks in flight per wave
    constexpr int NW = 4;
    __shared__ f32x4 red[NW][64];

    const int r = rows_by_nnz[blockIdx.x / PS];
    const int slice = blockIdx.x % PS;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int l16 = lane & 15, lq = lane >> 4;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(X, (uint32_t)M * K * 2);   // rows past M read as zero
    const uint32_t xoff = (uint32_t)(l16 * K + lq * 8) * 2;
    const uint32_t voff = (uint32_t)((slice * 16 + l16) * BS + lq * 8) * 2;

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int i1 = row_ptr[r + 1];
    for (int i = row_ptr[r] + wave; i < i1; i += NW * U) {
        bf16x8 a[U][KC], b[U][KC];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int iu = i + u * NW;
            const int ic = min(iu, i1 - 1);
            const uint32_t coff = (uint32_t)col_idx[ic] * BS * 2;
            const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + (size_t)ic * BS * BS, iu < i1 ? BS * BS * 2 : 0);
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                a[u][kc] = buf_load16(rv, voff + kc * 64, 0);
                b[u][kc] = buf_load16(rx, xoff + kc * 64, coff);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) acc = mfma(a[u][kc], b[u][kc], acc);
    }
    red[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {
        f32x4 v = red[0][lane];
#pragma unroll
        for (int w = 1; w < NW; ++w) v += red[w][lane];
        if (l16 < M) {
            const int n = r * BS + slice * 16 + lq * 4;
            if (bias) v = add_bias4(v, bias + n);
            store4_bf16(Y + (int64_t)l16 * N + n, v[0], v[1], v[2], v[3]);
        }
    }
}

// ------------------------------------------------------------------------------------------
// Weight gradient on the kept blocks (block-masked SDDMM): for block i of row r, column c,
//   dV[i][p][q] = sum_m dY[m][r*BS + p] * X[m][c*BS + q].
// Work-group = (run of up to GB kept blocks of one block row, chunk of M). Per stage of KM = 32*NW
// rows, the row's dY slab and the blocks' X slabs are staged in LDS in their natural layout
// (m-major) and read back transposed with ds_read_b64_tr_b16; wave w takes rows [32w, 32w+32) of
// the stage for every block of the run, so the dY fragments are loaded once per wave and reused
// by all blocks. Product orientation: A[q][k] = X[m][c*BS + q], B[k][p] = dY[m][r*BS + p], so
// D[q][p] = dV[p][q] and each lane holds 4 consecutive q of one p. The next stage's global loads
// run (into registers) while the current stage computes. At the end the waves' partial sums are
// added in LDS in wave order. With one chunk the sum is rounded to bf16 directly; otherwise fp32
// partials go to the workspace and k_dw_reduce adds them in chunk order.
// ------------------------------------------------------------------------------------------
template <int BS, int GB>
struct DwShape {
    static constexpr int NW = 4;
    static constexpr int KM = 32 * NW;           // rows per stage
    static constexpr int LD = BS + 8;            // padded slab pitch (elements)
    static constexpr int SLAB = KM * LD;         // elements per staged slab
    static constexpr int RLD = BS + 4;           // padded pitch of the reduction tile (floats)
    static constexpr size_t STAGE_BYTES = (size_t)(1 + GB) * SLAB * 2;
    static constexpr size_t RED_BYTES = (size_t)NW * BS * RLD * 4;
    static constexpr size_t LDS_BYTES = STAGE_BYTES > RED_BYTES ? STAGE_BYTES : RED_BYTES;
};

template <int BS, int GB>
__global__ __launch_bounds__(256) void k_dw(const uint16_t *__restrict__ dY, int N, const uint16_t *__restrict__ X,
                                            int K, int M, const int32_t *__restrict__ grp_row,
                                            const int32_t *__restrict__ grp_first, const int32_t *__restrict__ grp_count,
                                            const int32_t *__restrict__ col_idx, int mchunk, int nchunks, int nnzb,
                                            float *__restrict__ partial, uint16_t *__restrict__ dV) {
    using S = DwShape<BS, GB>;
    constexpr int NW = S::NW, KM = S::KM, LD = S::LD, SLAB = S::SLAB, RLD = S::RLD;
    constexpr int QT = BS / 16, PT = BS / 16;
    constexpr int CPR = BS / 8;                  // 16-byte chunks per slab row
    constexpr int CPS = KM * CPR / (NW * 64);    // chunks per thread per slab
    static_assert((KM * CPR) % (NW * 64) == 0, "slab staging must divide evenly");
    __shared__ __attribute__((aligned(16))) unsigned char smem[S::LDS_BYTES];
    uint16_t *sdy = reinterpret_cast<uint16_t *>(smem);   // [KM][LD]
    uint16_t *sx = sdy + SLAB;                             // [GB][KM][LD]

    const int gidx = blockIdx.x / nchunks, ch = blockIdx.x % nchunks;
    const int r = grp_row[gidx], i0 = grp_first[gidx], nb = grp_count[gidx];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, lq = lane >> 4;
    const int m_begin = ch * mchunk;
    const int m_end = min(M, m_begin + mchunk);

    int cofs[GB];
#pragma unroll
    for (int j = 0; j < GB; ++j) cofs[j] = (j < nb) ? col_idx[i0 + j] * BS : 0;

    f32x4 acc[GB][QT][PT];
#pragma unroll
    for (int j = 0; j < GB; ++j)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) acc[j][qt][pt] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 ry[CPS], rx[GB][CPS];
    // Stage rows [ms, ms + KM) of the dY slab and the X slabs; rows past m_end and absent blocks
    // read as zeros.
    auto load_stage = [&](int ms) __attribute__((always_inline)) {
        const uint32_t rows = (uint32_t)min(KM, m_end - ms);
        const __amdgpu_buffer_rsrc_t rdy = make_rsrc(dY + (int64_t)ms * N + r * BS, rows * N * 2);
        __amdgpu_buffer_rsrc_t rxs[GB];
#pragma unroll
        for (int j = 0; j < GB; ++j) rxs[j] = make_rsrc(X + (int64_t)ms * K + cofs[j], j < nb ? rows * K * 2 : 0);
#pragma unroll
        for (int k = 0; k < CPS; ++k) {
            const int e = tid + k * NW * 64, row = e / CPR, c8 = (e % CPR) * 8;
            ry[k] = buf_load16u(rdy, (uint32_t)(row * N + c8) * 2, 0);
#pragma unroll
            for (int j = 0; j < GB; ++j) rx[j][k] = buf_load16u(rxs[j], (uint32_t)(row * K + c8) * 2, 0);
        }
    };
    auto store_stage = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < CPS; ++k) {
            const int e = tid + k * NW * 64, row = e / CPR, c8 = (e % CPR) * 8;
            *reinterpret_cast<u32x4 *>(sdy + row * LD + c8) = ry[k];
#pragma unroll
            for (int j = 0; j < GB; ++j) *reinterpret_cast<u32x4 *>(sx + j * SLAB + row * LD + c8) = rx[j][k];
        }
    };

    if (m_begin < m_end) load_stage(m_begin);
    for (int ms = m_begin; ms < m_end; ms += KM) {
        __syncthreads();   // the previous stage's LDS reads are done
        store_stage();
        __syncthreads();
        if (ms + KM < m_end) load_stage(ms + KM);
        const int k0 = wave * 32 + lq * 8;
        bf16x8 bq[PT];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) bq[pt] = lds_read_tr8(sdy, LD, k0, pt * 16, l16);
#pragma unroll
        for (int j = 0; j < GB; ++j) {
            if (j >= nb) continue;
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) {
                const bf16x8 aq = lds_read_tr8(sx + j * SLAB, LD, k0, qt * 16, l16);
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) acc[j][qt][pt] = mfma(aq, bq[pt], acc[j][qt][pt]);
            }
        }
    }

    // Sum the waves' partials block by block: wave w writes red[w][p][q], then every thread adds
    // four consecutive q over w = 0..NW-1.
    float *red = reinterpret_cast<float *>(smem);
    constexpr int EPT = BS * BS / (NW * 64);   // output elements per thread per block
    for (int j = 0; j < nb; ++j) {
        __syncthreads();
#pragma unroll
        for (int jj = 0; jj < GB; ++jj) {
            if (jj != j) continue;
#pragma unroll
            for (int qt = 0; qt < QT; ++qt)
#pragma unroll
                for (int pt = 0; pt < PT; ++pt)
                    *reinterpret_cast<f32x4 *>(red + (wave * BS + pt * 16 + l16) * RLD + qt * 16 + lq * 4) =
                        acc[jj][qt][pt];
        }
        __syncthreads();
        const size_t blk = (size_t)(i0 + j) * BS * BS;
#pragma unroll
        for (int k = 0; k < EPT / 4; ++k) {
            const int e = (tid + k * NW * 64) * 4, p = e / BS, q = e % BS;
            f32x4 s = *reinterpret_cast<const f32x4 *>(red + p * RLD + q);
#pragma unroll
            for (int w = 1; w < NW; ++w) s += *reinterpret_cast<const f32x4 *>(red + (w * BS + p) * RLD + q);
            if (nchunks == 1)
                store4_bf16(dV + blk + e, s[0], s[1], s[2], s[3]);
            else
                *reinterpret_cast<f32x4 *>(partial + (size_t)ch * nnzb * BS * BS + blk + e) = s;
        }
    }
}

// Sums the per-chunk fp32 partials in chunk order and rounds to bf16 (4 elements per thread).
__global__ __launch_bounds__(256) void k_dw_reduce(const float *__restrict__ partial, int nchunks, size_t count,
                                                   uint16_t *__restrict__ dV) {
    const size_t e = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (e >= count) return;
    f32x4 s = *reinterpret_cast<const f32x4 *>(partial + e);
    for (int ch = 1; ch < nchunks; ++ch) s += *reinterpret_cast<const f32x4 *>(partial + (size_t)ch * count + e);
    store4_bf16(dV + e, s[0], s[1], s[2], s[3]);
}

// Bias gradient, pass 1: column sums of dY over one chunk of rows -> fp32 partials.
__global__ __launch_bounds__(256) void k_colsum_partial(const uint16_t *__restrict__ dY, int N, int64_t M,
                                                        int64_t rows_per, float *__restrict__ partial) {
    const int n = blockIdx.x * 256 + threadIdx.x;
    const int ch = blockIdx.y;
    if (n >= N) return;
    const int64_t m0 = (int64_t)ch * rows_per, m1 = std::min<int64_t>(M, m0 + rows_per);
    float s = 0.f;
    for (int64_t m = m0; m < m1; ++m) s += from_bf16(dY[m * N + n]);
    partial[(size_t)ch * N + n] = s;
}

// Bias gradient, pass 2: sum the partials in chunk order.
__global__ __launch_bounds__(256) void k_colsum_final(const float *__restrict__ partial, int nchunks, int N,
                                                      uint16_t *__restrict__ db) {
    const int n = blockIdx.x * 256 + threadIdx.x;
    if (n >= N) return;
    float s = 0.f;
    for (int ch = 0; ch < nchunks; ++ch) s += partial[(size_t)ch * N + n];
    db[n] = to_bf16(s);
}

__global__ __launch_bounds__(256) void k_fill_zero(uint16_t *__restrict__ p, size_t count) {
    const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (e < count) p[e] = 0;
}

// ---- host-side planning ----

// Tile shapes of the group GEMM: G output blocks x (NW*WM) activation rows per work-group.
enum Tile { TILE_WIDE = 0, TILE_NARROW = 1, TILE_SMALL = 2 };

int tile_override() {
    const char *s = std::getenv("BSR_GEMM_TILE");   // tuning knob: wide | narrow | small
    if (!s) return -1;
    if (!std::strcmp(s, "wide")) return TILE_WIDE;
    if (!std::strcmp(s, "narrow")) return TILE_NARROW;
    if (!std::strcmp(s, "small")) return TILE_SMALL;
    return -1;
}

// Picks the widest tile that still gives at least two work-groups per compute unit.
int choose_tile(const bsr_pattern &p, bool transposed, int64_t M) {
    const int forced = tile_override();
    if (forced >= 0) return forced;
    const GroupSchedule *s = transposed ? p.bwd : p.fwd;
    const int64_t want = 2 * kCUs;
    if ((int64_t)s[0].ngroups * ((M + 255) / 256) >= want) return TILE_WIDE;
    if ((int64_t)s[1].ngroups * ((M + 255) / 256) >= want) return TILE_NARROW;
    return TILE_SMALL;
}

struct DwPlan {
    int nchunks = 1;
    int mchunk = 0;
    int bchunks = 1;        // row chunks of the bias column sums
    int64_t brows = 0;
    size_t partial_bytes = 0, bias_off = 0, bias_bytes = 0, total = 0;
};

DwPlan plan_dw(const bsr_pattern &p, int64_t M) {
    DwPlan d;
    if (M <= 0) return d;
    constexpr int KM = 128;
    // enough work-groups for two per compute unit, without chunks shorter than 512 rows
    const int64_t ng = std::max(p.dw.ngroups, 1);
    const int64_t want = (2 * kCUs + ng - 1) / ng;
    const int64_t maxc = std::max<int64_t>(1, M / 512);
    d.nchunks = (int)std::max<int64_t>(1, std::min(want, maxc));
    d.mchunk = (int)(((M + d.nchunks - 1) / d.nchunks + KM - 1) / KM * KM);
    d.nchunks = (int)((M + d.mchunk - 1) / d.mchunk);
    d.bchunks = (int)std::min<int64_t>(64, std::max<int64_t>(1, M / 256));
    d.brows = (M + d.bchunks - 1) / d.bchunks;
    d.bchunks = (int)((M + d.brows - 1) / d.brows);
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    d.partial_bytes = d.nchunks > 1 ? (size_t)d.nchunks * p.nnzb * p.b * p.b * sizeof(float) : 0;
    d.bias_bytes = (size_t)d.bchunks * p.N * sizeof(float);
    d.bias_off = al(d.partial_bytes);
    d.total = d.bias_off + al(d.bias_bytes);
    return d;
}

int32_t launched(const char *what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(BSR_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
    return BSR_OK;
}

template <int BS, int G, int WM, bool TRANS>
void launch_gg(const bsr_pattern &p, int which, const FwdArgs &a, hipStream_t st) {
    constexpr int NW = 4, P = gemm_depth(BS);
    constexpr int BM = NW * WM;
    const DevSchedule &d = TRANS ? p.dev.bwd[which] : p.dev.fwd[which];
    const GroupSchedule &s = TRANS ? p.bwd[which] : p.fwd[which];
    const int nmtiles = (int)((a.M + BM - 1) / BM);
    const dim3 grid((unsigned)((int64_t)s.ngroups * nmtiles));
    hipLaunchKernelGGL((k_group_gemm<BS, G, WM, NW, P, TRANS>), grid, dim3(NW * 64), 0, st, a.act, a.in_ld, (int)a.M,
                       a.V, a.bias, a.out, a.out_ld, d.order, d.step_ptr, d.out, d.rec, d.hdr, nmtiles);
}

template <int BS, bool TRANS>
void launch_gg_tile(const bsr_pattern &p, int tile, const FwdArgs &a, hipStream_t st) {
    constexpr int GW = BS == 64 ? 4 : 8, GN = BS == 64 ? 2 : 4;
    if (tile == TILE_WIDE) launch_gg<BS, GW, 64, TRANS>(p, 0, a, st);
    else if (tile == TILE_NARROW) launch_gg<BS, GN, 64, TRANS>(p, 1, a, st);
    else launch_gg<BS, GN, 32, TRANS>(p, 1, a, st);
}

}  // namespace

int32_t launch_group_gemm(const bsr_pattern &p, bool transposed, const FwdArgs &a, void *stream) {
    const hipStream_t st = (hipStream_t)stream;
    const int tile = choose_tile(p, transposed, a.M);
    const int64_t nwg = (int64_t)(transposed ? p.bwd : p.fwd)[tile == TILE_WIDE ? 0 : 1].ngroups * ((a.M + 127) / 128);
    if (nwg > (int64_t)INT32_MAX) return fail(BSR_ERR_INVALID_ARG, "problem too large for one launch");
    if (p.b == 32) {
        if (transposed) launch_gg_tile<32, true>(p, tile, a, st);
        else launch_gg_tile<32, false>(p, tile, a, st);
    } else {
        if (transposed) launch_gg_tile<64, true>(p, tile, a, st);
        else launch_gg_tile<64, false>(p, tile, a, st);
    }
    return launched(transposed ? "bwd_input launch" : "fwd launch");
}

int32_t launch_small_m_fwd(const bsr_pattern &p, const FwdArgs &a, void *stream) {
    const hipStream_t st = (hipStream_t)stream;
    const DeviceMeta &d = p.dev;
    const dim3 grid((unsigned)(p.R * (p.b / 16)));
    if (p.b == 32)
        hipLaunchKernelGGL((k_small_m<32>), grid, dim3(256), 0, st, a.act, p.K, (int)a.M, a.V, a.bias, a.out, p.N,
                           d.row_ptr, d.col_idx, d.rows_by_nnz);
    else
        hipLaunchKernelGGL((k_small_m<64>), grid, dim3(256), 0, st, a.act, p.K, (int)a.M, a.V, a.bias, a.out, p.N,
                           d.row_ptr, d.col_idx, d.rows_by_nnz);
    return launched("fwd small-M launch");
}

size_t dw_workspace_bytes(const bsr_pattern &p, int64_t M) { return M > 0 ? plan_dw(p, M).total : 0; }

int32_t launch_dw(const bsr_pattern &p, const DwArgs &a, void *stream) {
    const hipStream_t st = (hipStream_t)stream;
    const DeviceMeta &d = p.dev;
    const size_t nval = (size_t)p.nnzb * p.b * p.b;
    if (a.M == 0) {
        if (nval) hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)((nval + 255) / 256)), dim3(256), 0, st, a.dV, nval);
        if (a.dbias)
            hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)((p.N + 255) / 256)), dim3(256), 0, st, a.dbias,
                               (size_t)p.N);
        return launched("bwd_weight zero fill");
    }
    const DwPlan pl = plan_dw(p, a.M);
    char *ws = static_cast<char *>(a.ws);
    float *partial = pl.nchunks > 1 ? reinterpret_cast<float *>(ws) : nullptr;
    if (p.nnzb > 0) {
        const dim3 grid((unsigned)((int64_t)p.dw.ngroups * pl.nchunks));
        if (p.b == 32)
            hipLaunchKernelGGL((k_dw<32, 4>), grid, dim3(256), 0, st, a.dY, p.N, a.X, p.K, (int)a.M, d.dw_row,
                               d.dw_first, d.dw_count, d.col_idx, pl.mchunk, pl.nchunks, p.nnzb, partial, a.dV);
        else
            hipLaunchKernelGGL((k_dw<64, 2>), grid, dim3(256), 0, st, a.dY, p.N, a.X, p.K, (int)a.M, d.dw_row,
                               d.dw_first, d.dw_count, d.col_idx, pl.mchunk, pl.nchunks, p.nnzb, partial, a.dV);
        if (pl.nchunks > 1)
            hipLaunchKernelGGL(k_dw_reduce, dim3((unsigned)((nval / 4 + 255) / 256)), dim3(256), 0, st, partial,
                               pl.nchunks, nval, a.dV);
    }
    if (a.dbias) {
        float *bp = reinterpret_cast<float *>(ws + pl.bias_off);
        hipLaunchKernelGGL(k_colsum_partial, dim3((unsigned)((p.N + 255) / 256), (unsigned)pl.bchunks), dim3(256), 0,
                           st, a.dY, p.N, a.M, pl.brows, bp);
        hipLaunchKernelGGL(k_colsum_final, dim3((unsigned)((p.N + 255) / 256)), dim3(256), 0, st, bp, pl.bchunks, p.N,
                           a.dbias);
    }
    return launched("bwd_weight launch");
}

}  // namespace bsr
