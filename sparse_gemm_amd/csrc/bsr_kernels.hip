// bsr_kernels.hip -- gfx950 (CDNA4) kernels of the block-sparse linear layer.
//
// Every kept b x b block is a real dense contraction, so each one runs on bf16 MFMA with fp32
// accumulation (pytorch_block_sparse summary page, "Technical Foundation": dense matrix-core
// products on the kept blocks, zero blocks skipped). Each output element is rounded once to bf16.
//
// Products use bf16 MFMA with fp32 accumulation (wave64):
//   v_mfma_f32_32x32x16_bf16 (the large-M kernels; on gfx950 it issues twice the flops per cycle of
//     the 16x16x32 form): lane l holds A[l%32][8*(l/32) + t] and B[8*(l/32) + t][l%32], t = 0..7;
//     result item v of lane l is D[8*(v/4) + 4*(l/32) + v%4][l%32].
//   v_mfma_f32_16x16x32_bf16 (small M): lane l holds A[l%16][8*(l/16) + t] and B[8*(l/16) + t][l%16];
//     result item v of lane l is D[4*(l/16) + v][l%16].
// Only the pairing of A's and B's k positions matters for the sum, so both operands always take
// the same k for the same (lane group, item).
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
typedef float f32x16 __attribute__((ext_vector_type(16)));
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

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 quad(const f32x16 &v, int q) { return f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]}; }

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

// 32x32x16 operand from a row-major T[k][n] tile (pitch ld elements) read transposed: lane l gets
// T[k0 + 8*(l/32) .. +7][n0 + l%32].
__device__ __forceinline__ bf16x8 lds_read_tr8_32(const uint16_t *tile, int ld, int k0, int n0, int lane) {
    const int gq = lane >> 4;
    return lds_read_tr8(tile, ld, k0 + (gq >> 1) * 8, n0 + (gq & 1) * 16, lane & 15);
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
// input gradient) and BM = NW * WM activation rows; wave w owns rows [w*WM, (w+1)*WM) for all G
// blocks, so every wave does the same work whatever blocks are present. A sub-step takes one
// input block of the activations (block column c of X, or block row r of dY) and up to S of the
// value blocks kept there (the host splits steps with more into several sub-steps):
//   out tile^T [n][m] += A[n][k] . B[k][m],   B[k][m] = act[m][in*BS + k]   (32x32x16 MFMA)
//   forward:    A[n][k] = V[i][n][k]   (natural layout, 16-byte LDS reads)
//   input grad: A[n][k] = V[i][k][n]   (transposed, ds_read_b64_tr_b16 of the natural layout)
// so each lane ends up with runs of 4 consecutive output columns of one activation row. Only kept blocks
// are loaded, once per work-group, into LDS slots; a sub-step first reads all its weight
// fragments, then runs the products of each member (uniform branches, static accumulators).
// Pipelining: at sub-step s the activation fragments and value blocks of sub-step s + P are
// loaded into registers (rings of P slots) while sub-step s computes; the value blocks of s + 1,
// loaded P - 1 sub-steps earlier, then go to the other half of a double-buffered LDS stage.
// Sub-step records are fetched by wave 0 into a small LDS ring one sub-step ahead of use. Every
// loop trip issues the same loads, so the compiler's wait counts stay exact.
// ------------------------------------------------------------------------------------------
template <int BS, int G, int S, int WM, int NW, int P, bool TRANS>
__global__ __launch_bounds__(NW * 64) void k_group_gemm(
    const uint16_t *__restrict__ act, int in_ld, int M, const uint16_t *__restrict__ V,
    const uint16_t *__restrict__ bias, uint16_t *__restrict__ out, int out_ld, const int32_t *__restrict__ order,
    const int32_t *__restrict__ sub_ptr, const int32_t *__restrict__ gout, const int32_t *__restrict__ rec,
    int nmtiles) {
    constexpr bool DIRECT = S == G;         // slot t feeds member t
    constexpr int NT = BS / 32;             // 32-wide output tiles per block
    constexpr int KC = BS / 16;             // 16-deep k chunks per block
    constexpr int MT = WM / 32;             // 32-row activation tiles per wave
    constexpr int BM = WM * NW;
    constexpr int LDW = BS + 8;             // padded LDS pitch of a staged block (elements)
    constexpr int NTH = NW * 64;
    constexpr int CPB = BS * BS / 8;        // 16-byte chunks per block
    constexpr int CPT = (S * CPB + NTH - 1) / NTH;   // chunks per thread per sub-step
    constexpr int RS = rec_stride(S);
    constexpr int RING = 4;                 // record ring entries in LDS
    static_assert(CPB % 64 == 0, "a wave's chunks must stay in one block");
    static_assert(RS <= 64, "one record word per lane");
    __shared__ __attribute__((aligned(16))) uint16_t wl[2][S][BS][LDW];   // staged blocks, by slot
    __shared__ __attribute__((aligned(16))) int32_t rring[RING][RS];

    // Work-groups are dispatched to the 8 XCDs round-robin; give each XCD a contiguous run of
    // logical tiles, ordered activation-tile-major, so that the groups sharing an activation tile
    // run together on one XCD and find it in that XCD's L2.
    const int ngroups = (int)(gridDim.x / nmtiles);
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int g = order[L % ngroups];
    const int mt0 = L / ngroups;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, lh = lane >> 5;
    const int mbase = mt0 * BM + wave * WM;
    const int rlane = min(lane, RS - 1);

    // Activations of this work-group's rows; rows past M read as zeros.
    const int rows = min(BM, M - mt0 * BM);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(act + (int64_t)mt0 * BM * in_ld, (uint32_t)rows * in_ld * 2);
    uint32_t voff[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) voff[mt] = (uint32_t)(((wave * WM + mt * 32 + l32) * in_ld + lh * 8) * 2);

    f32x16 acc[G][NT][MT];
#pragma unroll
    for (int t = 0; t < G; ++t)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[t][nt][mt][v] = 0.f;

    const int s0 = sub_ptr[g], s1 = sub_ptr[g + 1];
    bf16x8 xr[P][MT][KC];   // activation fragments of the next P sub-steps (ring)
    u32x4 wr[P][CPT];       // value-block chunks of the next P sub-steps (ring)
    int slot_of[P][S];      // slot words of the next P sub-steps (uniform)
    int rr[P];              // wave 0: records further ahead (ring; lane k holds word k)

    auto rec_at = [&](int sidx) __attribute__((always_inline)) {
        return rec[(size_t)min(sidx, s1 - 1) * RS + rlane];
    };
    auto load_x = [&](bf16x8(&slot)[MT][KC], int in_blk) __attribute__((always_inline)) {
        const uint32_t soff = (uint32_t)in_blk * BS * 2;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) slot[mt][kc] = buf_load16(ra, voff[mt] + kc * 32, soff);
    };
    // value block of a slot word
    auto blk_of = [](int word) __attribute__((always_inline)) { return DIRECT ? word : (word < 0 ? -1 : word >> 5); };
    auto load_w = [&](u32x4(&slot)[CPT], const int(&words)[S]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int k = (j * NTH + wave * 64) / CPB;   // slot: uniform per wave
            if (k >= S) continue;
            const int w = (tid + j * NTH) % CPB;
            const int blk = blk_of(words[k]);
            const __amdgpu_buffer_rsrc_t rw = make_rsrc(V + (size_t)max(blk, 0) * BS * BS, blk >= 0 ? BS * BS * 2 : 0);
            slot[j] = buf_load16u(rw, (uint32_t)w * 16, 0);
        }
    };
    // member fed by a slot word
    auto member_of = [](int k, int word) __attribute__((always_inline)) { return DIRECT ? k : (word & 31); };
    auto store_w = [&](int buf, const u32x4(&slot)[CPT]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int k = (j * NTH + wave * 64) / CPB;
            if (k >= S) continue;
            const int w = (tid + j * NTH) % CPB;
            *reinterpret_cast<u32x4 *>(&wl[buf][k][w / (BS / 8)][(w % (BS / 8)) * 8]) = slot[j];
        }
    };
    // All of the sub-step's weight fragments are read from LDS first (empty slots read stale data
    // that no product uses), then the products run member by member: for member t, every slot k
    // that feeds it (uniform tests), so each accumulator stays in its own registers.
    auto compute = [&](int buf, const bf16x8(&x)[MT][KC], const int(&words)[S]) __attribute__((always_inline)) {
        bf16x8 a[S][NT][KC];
#pragma unroll
        for (int k = 0; k < S; ++k)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) {
                    if constexpr (!TRANS)
                        a[k][nt][kc] = *reinterpret_cast<const bf16x8 *>(&wl[buf][k][nt * 32 + l32][kc * 16 + lh * 8]);
                    else
                        a[k][nt][kc] = lds_read_tr8_32(&wl[buf][k][0][0], LDW, kc * 16, nt * 32, lane);
                }
#pragma unroll
        for (int t = 0; t < G; ++t)
#pragma unroll
            for (int k = 0; k < S; ++k) {
                if (DIRECT && k != t) continue;
                if (words[k] < 0 || member_of(k, words[k]) != t) continue;   // uniform
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int kc = 0; kc < KC; ++kc)
                            acc[t][nt][mt] = mfma32(a[k][nt][kc], x[mt][kc], acc[t][nt][mt]);
            }
    };
    // record words from the LDS ring, all lanes reading the same entry
    auto ring_words = [&](int sidx, int &in_blk, int(&words)[S]) __attribute__((always_inline)) {
        const int32_t *e = rring[sidx % RING];
        in_blk = __builtin_amdgcn_readfirstlane(e[0]);
#pragma unroll
        for (int k = 0; k < S; ++k) words[k] = __builtin_amdgcn_readfirstlane(e[1 + k]);
    };

    if (s0 < s1) {
        // prologue: the first P sub-steps' records straight from memory, their loads, and the
        // record ring / wave 0's record registers set up as the loop expects at sub-step s0
#pragma unroll
        for (int u = 0; u < P; ++u) {
            const int r = rec_at(s0 + u);
            int words[S];
#pragma unroll
            for (int k = 0; k < S; ++k) words[k] = __builtin_amdgcn_readlane(r, 1 + k);
#pragma unroll
            for (int k = 0; k < S; ++k) slot_of[u][k] = words[k];
            load_x(xr[u], __builtin_amdgcn_readlane(r, 0));
            load_w(wr[u], words);
        }
        if (wave == 0) {
            if (lane < RS) rring[(s0 + P) % RING][lane] = rec_at(s0 + P);
#pragma unroll
            for (int v = 0; v < P; ++v) rr[v] = rec_at(s0 + (v == 0 ? 2 * P : P + v));
        }
        store_w(0, wr[0]);
        __builtin_amdgcn_s_waitcnt(0);   // drain: the loop's wait counts then hold on entry too
        __syncthreads();
        for (int s = s0; s < s1; s += P) {
#pragma unroll
            for (int u = 0; u < P; ++u) {
                const int cs = s + u;
                const int buf = (cs - s0) & 1;
                int in_next, words_next[S];
                ring_words(cs + P, in_next, words_next);       // record of sub-step cs + P
                load_w(wr[u], words_next);                      // its value blocks
                compute(buf, xr[u], slot_of[u]);
                load_x(xr[u], in_next);                         // its activations
#pragma unroll
                for (int k = 0; k < S; ++k) slot_of[u][k] = words_next[k];
                if (wave == 0) {                                // record of cs + P + 1 into the ring
                    if (lane < RS) rring[(cs + P + 1) % RING][lane] = rr[(u + 1) % P];
                    rr[(u + 1) % P] = rec_at(cs + 2 * P + 1);
                }
                store_w(buf ^ 1, wr[(u + 1) % P]);              // value blocks of sub-step cs + 1
                __syncthreads();
            }
        }
    }

    // Epilogue: item v of lane l is output column nt*32 + 8*(v/4) + 4*(l/32) + v%4 of the block,
    // activation row mt*32 + l%32 of the wave.
#pragma unroll
    for (int t = 0; t < G; ++t) {
        const int o = gout[g * G + t];
        if (o < 0) continue;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = mbase + mt * 32 + l32;
            if (m >= M) continue;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int n = o * BS + nt * 32 + q * 8 + lh * 4;
                    f32x4 v = quad(acc[t][nt][mt], q);
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
// Work-group = (item, chunk of M). An item is up to TR block rows x up to TC block columns (see
// DwSchedule); per stage of KM = 32*KCH rows, each row's dY slab and each column's X slab is staged
// once in LDS, in its natural m-major layout, and read back transposed with ds_read_b64_tr_b16.
// The NW waves tile the item's TR x TC grid in WR x WC sub-grids, so a wave's dY fragments serve its
// WC columns and its X fragments its WR rows. Product orientation (32x32x16 MFMA): A[q][k] =
// X[m][c*BS + q], B[k][p] = dY[m][r*BS + p], so D[q][p] = dV[p][q] and each lane holds runs of 4
// consecutive q of one p.
// Stages are prefetched D deep into registers (rows past the chunk and absent slabs read as zeros)
// and written to a double-buffered LDS stage one step ahead. FULL items multiply every block of
// the sub-grid (absent ones are products of real slabs but are never written): no branches around
// the products, for items that are mostly full. With one chunk of M the sums are
// rounded to bf16 directly; otherwise fp32 partials go to the workspace for k_dw_reduce.
// ------------------------------------------------------------------------------------------
template <int BS, int TR, int TC, int WR, int WC, int KCH, int D, bool FULL, int NW>
__global__ __launch_bounds__(NW * 64) void k_dw_tile(const uint16_t *__restrict__ dY, int N,
                                                 const uint16_t *__restrict__ X, int K, int M,
                                                 const int32_t *__restrict__ items, int mchunk, int nchunks,
                                                 const int32_t *__restrict__ cmap, int nkind,
                                                 float *__restrict__ partial, uint16_t *__restrict__ dV) {
    constexpr int NTH = NW * 64;
    constexpr int WCOLS = TC / WC;            // waves along the item's columns
    static_assert((TR / WR) * WCOLS == NW && TR % WR == 0 && TC % WC == 0, "waves must tile the item");
    constexpr int NS = TR + TC;               // staged slabs: dY rows first, then X columns
    constexpr int KM = 32 * KCH;              // rows per stage
    constexpr int LD = BS + 8;                // padded slab pitch (elements)
    constexpr int CPS = KM * BS / 8;          // 16-byte chunks per slab
    constexpr int LPT = (NS * CPS + NTH - 1) / NTH;   // loads per thread per stage
    static_assert(CPS % 64 == 0, "a wave's chunks must stay in one slab");
    constexpr int QT = BS / 32, PT = BS / 32;   // 32x32 output tiles per block
    constexpr int TS = DwShape{TR, TC}.TS();
    __shared__ __attribute__((aligned(16))) uint16_t lds[2][NS][KM][LD];

    const int item = blockIdx.x / nchunks, ch = blockIdx.x % nchunks;
    const int32_t *it = items + (size_t)item * TS;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, lh = lane >> 5;
    const int wr = wave / WCOLS, wc = wave % WCOLS;
    const int m_begin = ch * mchunk;
    const int m_end = min(M, m_begin + mchunk);
    const int nst = ((m_end - m_begin + KM - 1) / KM + D - 1) / D * D;

    // This thread's staging chunks: slab (uniform per wave: a dY row first, then X columns) and
    // its byte offset inside the slab.
    int sid[LPT];
    uint32_t svoff[LPT];
#pragma unroll
    for (int j = 0; j < LPT; ++j) {
        const int slab = (j * NTH + wave * 64) / CPS;
        const int w = (tid + j * NTH) % CPS, row = w / (BS / 8), c8 = (w % (BS / 8)) * 8;
        sid[j] = slab < NS ? it[slab] : -1;
        svoff[j] = (uint32_t)(row * (slab < TR ? N : K) + c8) * 2;
    }
    // kept blocks of this wave's sub-grid: bit i*WC + j
    uint32_t present = 0;
#pragma unroll
    for (int i = 0; i < WR; ++i)
#pragma unroll
        for (int j = 0; j < WC; ++j)
            if (it[TR + TC + (wr * WR + i) * TC + wc * WC + j] >= 0) present |= 1u << (i * WC + j);

    f32x16 acc[WR][WC][QT][PT];
#pragma unroll
    for (int i = 0; i < WR; ++i)
#pragma unroll
        for (int j = 0; j < WC; ++j)
#pragma unroll
            for (int qt = 0; qt < QT; ++qt)
#pragma unroll
                for (int pt = 0; pt < PT; ++pt)
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[i][j][qt][pt][v] = 0.f;

    u32x4 ring[D][LPT];
    auto load_stage = [&](u32x4(&slot)[LPT], int st) __attribute__((always_inline)) {
        const int ms = m_begin + st * KM;
        const int rows = max(0, min(KM, m_end - ms));
#pragma unroll
        for (int j = 0; j < LPT; ++j) {
            const int slab = (j * NTH + wave * 64) / CPS;
            const int ld = slab < TR ? N : K;
            const bool ok = sid[j] >= 0 && rows > 0;
            const uint16_t *base = (slab < TR ? dY : X) + (int64_t)ms * ld + (int64_t)max(sid[j], 0) * BS;
            const __amdgpu_buffer_rsrc_t r = make_rsrc(ok ? base : dY, ok ? (uint32_t)rows * ld * 2 : 0);
            slot[j] = buf_load16u(r, svoff[j], 0);
        }
    };
    auto store_stage = [&](int buf, const u32x4(&slot)[LPT]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < LPT; ++j) {
            const int slab = (j * NTH + wave * 64) / CPS;
            if (slab >= NS) continue;   // uniform per wave
            const int w = (tid + j * NTH) % CPS, row = w / (BS / 8), c8 = (w % (BS / 8)) * 8;
            *reinterpret_cast<u32x4 *>(&lds[buf][slab][row][c8]) = slot[j];
        }
    };
    auto compute = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < 2 * KCH; ++kk) {   // 16 rows of the stage per product
            const int k0 = kk * 16;
            bf16x8 bq[WR][PT];
#pragma unroll
            for (int i = 0; i < WR; ++i)
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) bq[i][pt] = lds_read_tr8_32(&lds[buf][wr * WR + i][0][0], LD, k0, pt * 32, lane);
#pragma unroll
            for (int j = 0; j < WC; ++j) {
                uint32_t colmask = 0;
#pragma unroll
                for (int i = 0; i < WR; ++i) colmask |= 1u << (i * WC + j);
                if (!FULL && !(present & colmask)) continue;   // uniform per wave
                bf16x8 aq[QT];
#pragma unroll
                for (int qt = 0; qt < QT; ++qt)
                    aq[qt] = lds_read_tr8_32(&lds[buf][TR + wc * WC + j][0][0], LD, k0, qt * 32, lane);
#pragma unroll
                for (int i = 0; i < WR; ++i) {
                    if (!FULL && !((present >> (i * WC + j)) & 1)) continue;
#pragma unroll
                    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
                        for (int pt = 0; pt < PT; ++pt) acc[i][j][qt][pt] = mfma32(aq[qt], bq[i][pt], acc[i][j][qt][pt]);
                }
            }
        }
    };

#pragma unroll
    for (int u = 0; u < D; ++u) load_stage(ring[u], u);
    store_stage(0, ring[0]);
    __builtin_amdgcn_s_waitcnt(0);   // drain: the loop's wait counts then hold on entry too
    __syncthreads();
    for (int st = 0; st < nst; st += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            const int cs = st + u;
            const int buf = cs & 1;
            compute(buf);
            store_stage(buf ^ 1, ring[(u + 1) % D]);   // stage cs + 1, loaded D - 1 stages ago
            load_stage(ring[u], cs + D);
            __syncthreads();
        }
    }

    // Write the blocks: item v of lane l is q = qt*32 + 8*(v/4) + 4*(l/32) + v%4, p = pt*32 + l%32.
#pragma unroll
    for (int i = 0; i < WR; ++i)
#pragma unroll
        for (int j = 0; j < WC; ++j) {
            const int e = it[TR + TC + (wr * WR + i) * TC + wc * WC + j];
            if (e < 0) continue;
#pragma unroll
            for (int qt = 0; qt < QT; ++qt)
#pragma unroll
                for (int pt = 0; pt < PT; ++pt)
#pragma unroll
                    for (int vq = 0; vq < 4; ++vq) {
                        const int in = (pt * 32 + l32) * BS + qt * 32 + vq * 8 + lh * 4;
                        const f32x4 v = quad(acc[i][j][qt][pt], vq);
                        if (nchunks == 1)
                            store4_bf16(dV + (size_t)e * BS * BS + in, v[0], v[1], v[2], v[3]);
                        else
                            *reinterpret_cast<f32x4 *>(partial + ((size_t)ch * nkind + cmap[e]) * BS * BS + in) = v;
                    }
        }
}

// ------------------------------------------------------------------------------------------
// Weight gradient, runs: an item of one block row r and up to GB of its kept blocks (columns
// cols[j], CSR index blk[j]). Per stage of KM = 32*NW rows, the row's dY slab and the blocks' X
// slabs are staged in LDS (m-major) and read back transposed; wave w takes rows [32w, 32w + 32)
// of the stage for every block of the run, so its dY fragments serve all the run's blocks. The
// next stage's loads (rows past the chunk and absent blocks read as zeros) are issued into
// registers before the current stage computes. At the end the waves' partial sums are added in
// LDS in wave order. Orientation and output as in k_dw_tile.
// ------------------------------------------------------------------------------------------
template <int BS, int GB>
struct DwRunShape {
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
__global__ __launch_bounds__(256) void k_dw_runs(const uint16_t *__restrict__ dY, int N,
                                                 const uint16_t *__restrict__ X, int K, int M,
                                                 const int32_t *__restrict__ items, int mchunk, int nchunks,
                                                 const int32_t *__restrict__ cmap, int nkind,
                                                 float *__restrict__ partial, uint16_t *__restrict__ dV) {
    using S = DwRunShape<BS, GB>;
    constexpr int NW = S::NW, KM = S::KM, LD = S::LD, SLAB = S::SLAB, RLD = S::RLD;
    constexpr int QT = BS / 32, PT = BS / 32;   // 32x32 output tiles per block
    constexpr int CPR = BS / 8;                  // 16-byte chunks per slab row
    constexpr int CPS = KM * CPR / (NW * 64);    // chunks per thread per slab
    constexpr int TS = DwShape{1, GB}.TS();
    static_assert((KM * CPR) % (NW * 64) == 0, "slab staging must divide evenly");
    __shared__ __attribute__((aligned(16))) unsigned char smem[S::LDS_BYTES];
    uint16_t *sdy = reinterpret_cast<uint16_t *>(smem);   // [KM][LD]
    uint16_t *sx = sdy + SLAB;                             // [GB][KM][LD]

    const int item = blockIdx.x / nchunks, ch = blockIdx.x % nchunks;
    const int32_t *it = items + (size_t)item * TS;
    const int r = it[0];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, lh = lane >> 5;
    const int m_begin = ch * mchunk;
    const int m_end = min(M, m_begin + mchunk);

    int col[GB];
    uint32_t present = 0;
#pragma unroll
    for (int j = 0; j < GB; ++j) {
        col[j] = it[1 + j];
        if (it[1 + GB + j] >= 0) present |= 1u << j;
    }

    f32x16 acc[GB][QT][PT];
#pragma unroll
    for (int j = 0; j < GB; ++j)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
#pragma unroll
            for (int pt = 0; pt < PT; ++pt)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[j][qt][pt][v] = 0.f;

    u32x4 ry[CPS], rx[GB][CPS];
    auto load_stage = [&](int ms) __attribute__((always_inline)) {
        const uint32_t rows = (uint32_t)max(0, min(KM, m_end - ms));
        const __amdgpu_buffer_rsrc_t rdy = make_rsrc(dY + (int64_t)ms * N + r * BS, rows * N * 2);
#pragma unroll
        for (int k = 0; k < CPS; ++k) {
            const int e = tid + k * NW * 64, row = e / CPR, c8 = (e % CPR) * 8;
            ry[k] = buf_load16u(rdy, (uint32_t)(row * N + c8) * 2, 0);
        }
#pragma unroll
        for (int j = 0; j < GB; ++j) {
            const bool ok = col[j] >= 0;
            const __amdgpu_buffer_rsrc_t rxj =
                make_rsrc(X + (int64_t)ms * K + (int64_t)max(col[j], 0) * BS, ok ? rows * K * 2 : 0);
#pragma unroll
            for (int k = 0; k < CPS; ++k) {
                const int e = tid + k * NW * 64, row = e / CPR, c8 = (e % CPR) * 8;
                rx[j][k] = buf_load16u(rxj, (uint32_t)(row * K + c8) * 2, 0);
            }
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

    load_stage(m_begin);
    for (int ms = m_begin; ms < m_end; ms += KM) {
        __syncthreads();   // the previous stage's LDS reads are done
        store_stage();
        __syncthreads();
        load_stage(ms + KM);   // past the chunk: zeros, never used
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {   // this wave's 32 rows, 16 per product
            const int k0 = wave * 32 + kk * 16;
            bf16x8 bq[PT];
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) bq[pt] = lds_read_tr8_32(sdy, LD, k0, pt * 32, lane);
#pragma unroll
            for (int j = 0; j < GB; ++j) {
                if (!((present >> j) & 1)) continue;   // uniform
#pragma unroll
                for (int qt = 0; qt < QT; ++qt) {
                    const bf16x8 aq = lds_read_tr8_32(sx + j * SLAB, LD, k0, qt * 32, lane);
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) acc[j][qt][pt] = mfma32(aq, bq[pt], acc[j][qt][pt]);
                }
            }
        }
    }

    // Sum the waves' partials block by block: wave w writes red[w][p][q], then every thread adds
    // four consecutive q over w = 0..NW-1.
    float *red = reinterpret_cast<float *>(smem);
    constexpr int EPT = BS * BS / (NW * 64);   // output elements per thread per block
#pragma unroll
    for (int j = 0; j < GB; ++j) {
        const int e_blk = it[1 + GB + j];
        if (e_blk < 0) continue;   // uniform
        __syncthreads();
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
#pragma unroll
            for (int pt = 0; pt < PT; ++pt)
#pragma unroll
                for (int vq = 0; vq < 4; ++vq)
                    *reinterpret_cast<f32x4 *>(red + (wave * BS + pt * 32 + l32) * RLD + qt * 32 + vq * 8 + lh * 4) =
                        quad(acc[j][qt][pt], vq);
        __syncthreads();
#pragma unroll
        for (int k = 0; k < EPT / 4; ++k) {
            const int e = (tid + k * NW * 64) * 4, p = e / BS, q = e % BS;
            f32x4 sum = *reinterpret_cast<const f32x4 *>(red + p * RLD + q);
#pragma unroll
            for (int w = 1; w < NW; ++w) sum += *reinterpret_cast<const f32x4 *>(red + (w * BS + p) * RLD + q);
            if (nchunks == 1)
                store4_bf16(dV + (size_t)e_blk * BS * BS + e, sum[0], sum[1], sum[2], sum[3]);
            else
                *reinterpret_cast<f32x4 *>(partial + ((size_t)ch * nkind + cmap[e_blk]) * BS * BS + e) = sum;
        }
    }
}

// Sums the per-chunk fp32 partials of one kind of work item in chunk order and rounds to bf16
// (4 elements per thread). partial is [nchunks][nblocks][bb]; block k of the kind is CSR block
// blocks[k].
__global__ __launch_bounds__(256) void k_dw_reduce(const float *__restrict__ partial, int nchunks,
                                                   const int32_t *__restrict__ blocks, int nblocks, int bb,
                                                   uint16_t *__restrict__ dV) {
    const size_t e = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
    const size_t count = (size_t)nblocks * bb;
    if (e >= count) return;
    f32x4 s = *reinterpret_cast<const f32x4 *>(partial + e);
    for (int ch = 1; ch < nchunks; ++ch) s += *reinterpret_cast<const f32x4 *>(partial + (size_t)ch * count + e);
    const size_t k = e / bb;
    store4_bf16(dV + (size_t)blocks[k] * bb + (e - k * bb), s[0], s[1], s[2], s[3]);
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

// Tile of a group GEMM call: which of the pattern's two group schedules (wide G or narrow G)
// and how many waves (32 activation rows each) per work-group.
struct GemmTile {
    int k = 0;    // 0 = wide groups, 1 = narrow groups
    int nw = kGemmWaves;
};

// The widest tile that still gives every compute unit at least two work-groups (so that one
// work-group's prologue and epilogue overlap another's main loop): wide groups of 8 waves, then
// narrow groups of 8 waves, else narrow groups of 4 waves.
GemmTile choose_tile(const bsr_pattern &p, bool transposed, int64_t M) {
    const char *f = std::getenv("BSR_GEMM_TILE");   // tuning knob: wide | narrow | small
    if (f && !std::strcmp(f, "wide")) return GemmTile{0, kGemmWaves};
    if (f && !std::strcmp(f, "narrow")) return GemmTile{1, kGemmWaves};
    if (f && !std::strcmp(f, "small")) return GemmTile{1, kGemmWavesSmall};
    const GroupSchedule *s = transposed ? p.bwd : p.fwd;
    const int64_t nmt = (M + gemm_rows(p.b) - 1) / gemm_rows(p.b);
    if ((int64_t)s[0].ngroups * nmt >= 2 * kCUs) return GemmTile{0, kGemmWaves};
    if ((int64_t)s[1].ngroups * nmt >= 2 * kCUs) return GemmTile{1, kGemmWaves};
    return GemmTile{1, kGemmWavesSmall};
}

// M-split of one kind of weight-gradient item.
struct DwSplit {
    int nchunks = 1, mchunk = 0;
    size_t off = 0, bytes = 0;   // fp32 partials in the workspace (only when nchunks > 1)
};

struct DwPlan {
    DwSplit dense, runs;
    int bchunks = 1;        // row chunks of the bias column sums
    int64_t brows = 0;
    size_t bias_off = 0, bias_bytes = 0, total = 0;
};

// Enough chunks of M for `slots` work-groups from n items, chunks of at least min_rows rows
// (each split costs an fp32 partial of the kind's blocks).
DwSplit split_m(int64_t M, int n, int64_t slots, int64_t min_rows) {
    DwSplit s;
    if (n <= 0) return s;
    const int64_t want = (slots + n - 1) / n;
    const int64_t maxc = std::max<int64_t>(1, M / min_rows);
    s.nchunks = (int)std::max<int64_t>(1, std::min(want, maxc));
    s.mchunk = (int)(((M + s.nchunks - 1) / s.nchunks + 127) / 128 * 128);
    s.nchunks = (int)((M + s.mchunk - 1) / s.mchunk);
    return s;
}

DwPlan plan_dw(const bsr_pattern &p, int64_t M) {
    DwPlan d;
    if (M <= 0) return d;
    // dense items: one 8-wave work-group per CU; runs: three 4-wave work-groups per CU
    d.dense = split_m(M, p.dw.dense.n, kCUs, 256);
    d.runs = split_m(M, p.dw.runs.n, 3 * kCUs, 512);
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    const size_t bb = (size_t)p.b * p.b * sizeof(float);
    d.dense.bytes = d.dense.nchunks > 1 ? (size_t)d.dense.nchunks * p.dw.dense_blocks.size() * bb : 0;
    d.runs.bytes = d.runs.nchunks > 1 ? (size_t)d.runs.nchunks * p.dw.run_blocks.size() * bb : 0;
    d.dense.off = 0;
    d.runs.off = al(d.dense.bytes);
    d.bchunks = (int)std::min<int64_t>(64, std::max<int64_t>(1, M / 256));
    d.brows = (M + d.bchunks - 1) / d.bchunks;
    d.bchunks = (int)((M + d.brows - 1) / d.brows);
    d.bias_bytes = (size_t)d.bchunks * p.N * sizeof(float);
    d.bias_off = d.runs.off + al(d.runs.bytes);
    d.total = d.bias_off + al(d.bias_bytes);
    return d;
}

int32_t launched(const char *what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(BSR_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
    return BSR_OK;
}

template <int BS, int G, int S, int NW, bool TRANS>
void launch_gg(const GroupSchedule &s, const DevSchedule &d, const FwdArgs &a, hipStream_t st) {
    constexpr int WM = gemm_wave_rows(BS), P = gemm_depth(BS, G, S), BM = NW * WM;
    const int nmtiles = (int)((a.M + BM - 1) / BM);
    const dim3 grid((unsigned)((int64_t)s.ngroups * nmtiles));
    hipLaunchKernelGGL((k_group_gemm<BS, G, S, WM, NW, P, TRANS>), grid, dim3(NW * 64), 0, st, a.act, a.in_ld,
                       (int)a.M, a.V, a.bias, a.out, a.out_ld, d.order, d.sub_ptr, d.out, d.rec, nmtiles);
}

// Dispatch on the block size, the schedule's (G, S) and the waves per work-group to the
// instantiated kernels (see gemm_slot_options; narrow groups also have the 4-wave form).
template <bool TRANS>
int32_t launch_gg_shape(const bsr_pattern &p, const GroupSchedule &s, const DevSchedule &d, int nw,
                        const FwdArgs &a, hipStream_t st) {
    const int key = (p.b * 10000 + s.G * 100 + s.S) * 10 + (nw == kGemmWaves ? 0 : 1);
    constexpr int W8 = kGemmWaves, W4 = kGemmWavesSmall;
    switch (key) {
        case 3208020: launch_gg<32, 8, 2, W8, TRANS>(s, d, a, st); break;
        case 3208040: launch_gg<32, 8, 4, W8, TRANS>(s, d, a, st); break;
        case 3208080: launch_gg<32, 8, 8, W8, TRANS>(s, d, a, st); break;
        case 3204020: launch_gg<32, 4, 2, W8, TRANS>(s, d, a, st); break;
        case 3204040: launch_gg<32, 4, 4, W8, TRANS>(s, d, a, st); break;
        case 3204021: launch_gg<32, 4, 2, W4, TRANS>(s, d, a, st); break;
        case 3204041: launch_gg<32, 4, 4, W4, TRANS>(s, d, a, st); break;
        case 6402010: launch_gg<64, 2, 1, W8, TRANS>(s, d, a, st); break;
        case 6402020: launch_gg<64, 2, 2, W8, TRANS>(s, d, a, st); break;
        case 6401010: launch_gg<64, 1, 1, W8, TRANS>(s, d, a, st); break;
        case 6401011: launch_gg<64, 1, 1, W4, TRANS>(s, d, a, st); break;
        default: return fail(BSR_ERR_UNSUPPORTED, "no kernel for this group shape");
    }
    return BSR_OK;
}

}  // namespace

int32_t launch_group_gemm(const bsr_pattern &p, bool transposed, const FwdArgs &a, void *stream) {
    const hipStream_t st = (hipStream_t)stream;
    const GemmTile t = choose_tile(p, transposed, a.M);
    const GroupSchedule &s = (transposed ? p.bwd : p.fwd)[t.k];
    const DevSchedule &d = (transposed ? p.dev.bwd : p.dev.fwd)[t.k];
    const int rows = t.nw * gemm_wave_rows(p.b);
    const int64_t nwg = (int64_t)s.ngroups * ((a.M + rows - 1) / rows);
    if (nwg > (int64_t)INT32_MAX) return fail(BSR_ERR_INVALID_ARG, "problem too large for one launch");
    const int32_t rc = transposed ? launch_gg_shape<true>(p, s, d, t.nw, a, st) : launch_gg_shape<false>(p, s, d, t.nw, a, st);
    if (rc != BSR_OK) return rc;
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
    if (p.nnzb > 0) {
        const DwArgs &x = a;
        auto launch = [&](auto kernel, int nthreads, int n, const int32_t *items, const DwSplit &sp, int nkind) {
            if (n == 0) return;
            float *partial = sp.nchunks > 1 ? reinterpret_cast<float *>(ws + sp.off) : nullptr;
            hipLaunchKernelGGL(kernel, dim3((unsigned)((int64_t)n * sp.nchunks)), dim3(nthreads), 0, st, x.dY, p.N, x.X,
                               p.K, (int)x.M, items, sp.mchunk, sp.nchunks, d.dw_cmap, nkind, partial, x.dV);
        };
        const int nd = (int)p.dw.dense_blocks.size(), nr = (int)p.dw.run_blocks.size();
        if (p.b == 32) {
            launch(k_dw_tile<32, 8, 8, 4, 2, 1, 2, true, 8>, 512, p.dw.dense.n, d.dw_dense, pl.dense, nd);
            launch(k_dw_runs<32, 4>, 256, p.dw.runs.n, d.dw_runs, pl.runs, nr);
        } else {
            launch(k_dw_tile<64, 4, 4, 2, 1, 1, 2, true, 8>, 512, p.dw.dense.n, d.dw_dense, pl.dense, nd);
            launch(k_dw_runs<64, 2>, 256, p.dw.runs.n, d.dw_runs, pl.runs, nr);
        }
        const int bb = p.b * p.b;
        auto reduce = [&](const DwSplit &sp, const int32_t *blocks, int nblk) {
            if (sp.nchunks <= 1 || nblk == 0) return;
            const size_t count = (size_t)nblk * bb;
            hipLaunchKernelGGL(k_dw_reduce, dim3((unsigned)((count / 4 + 255) / 256)), dim3(256), 0, st,
                               reinterpret_cast<const float *>(ws + sp.off), sp.nchunks, blocks, nblk, bb, a.dV);
        };
        reduce(pl.dense, d.dw_dense_blocks, nd);
        reduce(pl.runs, d.dw_run_blocks, nr);
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
