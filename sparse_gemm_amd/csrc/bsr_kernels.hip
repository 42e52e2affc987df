// bsr_kernels.hip -- gfx950 (CDNA4) kernels of the block-sparse linear layer.
//
// Every kept b x b block is a real dense contraction, so each one runs on bf16 MFMA with fp32
// accumulation (pytorch_block_sparse summary page, "Technical Foundation": dense matrix-core
// products on the kept blocks, zero blocks skipped). Each output element is rounded once to bf16.
//
// Matrix-core operand layouts and the transposing LDS read are described in bsr_device.hpp.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "bsr_device.hpp"
#include "bsr_internal.hpp"

namespace bsr {
namespace {

using namespace dev;

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 buf_load16u(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}


// ------------------------------------------------------------------------------------------
// Panel GEMM: forward (TRANS = false) and input gradient (TRANS = true).
//
// A work-group owns G output blocks (block rows of W for the forward, block columns for the
// input gradient) and BM = 32 * NW activation rows; compute wave w owns rows [32 w, 32 w + 32)
// for all G blocks. The activations are read in panels of 64 columns: one full 128-byte cache
// line per row, which is what the load path of a CU serves best (it handles a bounded number of
// distinct cache lines per clock, however few of their bytes are used). A sub-step stages one
// panel of the work-group's rows and up to S kept value blocks of that panel in LDS, then every
// compute wave runs the products of each unit (a member's kept block inside the panel) that has
// a block:
//   out tile^T [n][m] += A[n][k] . B[k][m],   B[k][m] = act[m][panel*64 + k]   (32x32x16 MFMA)
//   forward:    A[n][k] = V[i][n][k]   (natural layout, 16-byte LDS reads)
//   input grad: A[n][k] = V[i][k][n]   (transposed, ds_read_b64_tr_b16 of the natural layout)
// so each lane ends up with runs of 4 consecutive output columns of one activation row.
// The loads go straight from memory to LDS, NST stages deep (D = NST - 1 sub-steps ahead), and are
// issued by NL extra loader waves, so that the compute waves never stall behind a full load queue
// and loads overlap the products. Sub-step s: loaders wait for their loads of s, then a barrier
// (the stage of s is complete; nobody reads the stage of s - 1 any more), then the loaders issue
// the loads of s + D into the stage of s - 1 while the compute waves run the products of s. In
// each stage the 16-byte chunks of every row are XOR swizzled so that operand reads are free of
// bank conflicts.
// ------------------------------------------------------------------------------------------

// SP: the form of the value blocks (forward only): kDense bf16 blocks, kImage24 2:4 block images
// (bsr_values_pack_24), kCompact24 the compressed 2:4 form as it is (kept values V [nnzb][BS][BS/2],
// index words meta [nnzb][BS][BS/16]).
constexpr int kDense = 0, kImage24 = 1, kCompact24 = 2;
template <int BS, int G, int S, int NW, int NL, int NST, int MS, bool TRANS, int SP = kDense>
__global__ __launch_bounds__((NW + NL) * 64) void k_panel_gemm(
    const uint16_t *__restrict__ act, int in_ld, int M, const uint16_t *__restrict__ V, uint32_t v_bytes,
    const uint16_t *__restrict__ meta, uint32_t m_bytes,
    const uint16_t *__restrict__ bias, uint16_t *__restrict__ out, int out_ld, const int32_t *__restrict__ order,
    const int32_t *__restrict__ sub_ptr, const int32_t *__restrict__ gout, const int32_t *__restrict__ rec,
    int ngroups, int nmtiles, int tpc) {
    constexpr int PB = kPanelCols / BS;     // blocks per panel
    constexpr int U = G * PB;               // units per panel
    constexpr int NT = BS / 32;             // 32-wide output tiles per block
    constexpr int KCB = BS / 16;            // 16-deep k chunks per block
    constexpr int BM = NW * 32;             // activation rows per work-group
    // Compute wave w takes RW = MS tiles of 32 rows and GW = G / MS members: rows
    // [wr * 32 * MS, + 32 * MS) and members [wm * GW, + GW) with wr = w % (NW / MS), wm = w / (NW / MS).
    // With MS = 2 every value fragment read from LDS feeds two products (one per row tile).
    constexpr int RW = MS, GW = G / MS;
    static_assert(G % MS == 0 && NW % MS == 0, "member split");
    constexpr int XB = BM * 128;            // bytes of a staged activation panel
    constexpr int RB = BS * 2;              // bytes per row of a value block
    constexpr int WBB = BS * RB;            // bytes per value block
    constexpr int STAGE = XB + S * WBB + kRecInts * 4;   // activations, value blocks, a record
    constexpr int D = NST - 1;              // sub-steps in flight ahead of the one computed
    static_assert(NST == 2 || NST == 3, "two or three stages");
    constexpr int CPS = WBB / 1024;         // 1 KB load chunks per block
    // compressed 2:4 blocks in a slot of WBB bytes: the kept values (rows of BS bytes) in its first
    // CB bytes (chunks 0 .. CB / 1024 - 1), the index words (rows of BS / 8 bytes) in the MB bytes
    // after them (chunk CB / 1024, lanes below MB / 16); the slot's remaining chunks load nothing
    constexpr int CB = BS * BS, MB = BS * BS / 8;
    static_assert(SP != kCompact24 || (!TRANS && CB + 1024 <= WBB), "compressed slot layout");
    constexpr int XPL = BM / 8 / NL;        // activation loads (8 rows x 128 bytes) per loader wave
    constexpr int WPL = S * CPS / NL;       // value-block chunks per loader wave
    constexpr int MAXL = XPL + WPL + 1;     // loads per loader wave and sub-step, at most
    static_assert(BM / 8 % NL == 0 && S * CPS % NL == 0, "loads must spread evenly over the loader waves");
    static_assert(U <= 16 && S <= 8, "unit map: 16 units of 4 bits, slots below 15");
    static_assert(2 * MAXL <= 63, "vmcnt range");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[NST * STAGE];

    // Work-group -> (group, activation tile). Each XCD takes a contiguous run of logical indices
    // (work-groups are dealt to the XCDs round-robin); logical indices run over chunks of tpc
    // activation tiles, and inside a chunk over the groups (most sub-steps first), then the tiles.
    // So every XCD gets all groups of its tiles (balanced work), and the work-groups running
    // together on one XCD share a few activation tiles (their panels) and their groups' value
    // blocks through that XCD's L2.
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int chunk = L / (tpc * ngroups), r4 = L % (tpc * ngroups);
    const int mc = min(tpc, nmtiles - tpc * chunk);   // tiles in this chunk
    const int g = order[r4 / mc];
    const int mt0 = tpc * chunk + r4 % mc;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool loader = wave >= NW;
    const int lw = wave - NW;               // loader index (loader waves only)
    const int wr = wave % (NW / MS), wm = wave / (NW / MS);   // compute waves: row group, member group
    const int l32 = lane & 31, lh = lane >> 5;

    // Activations of this work-group's rows; rows past M read as zeros.
    const int rows = min(BM, M - mt0 * BM);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(act + (int64_t)mt0 * BM * in_ld, (uint32_t)rows * in_ld * 2);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(V, v_bytes);
    const __amdgpu_buffer_rsrc_t rm = make_rsrc(meta, m_bytes);
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(rec, (uint32_t)sub_ptr[ngroups] * kRecInts * 4);
    const uint32_t sbase = lds_addr(smem);
    // loader lw's activation load i stages tile rows 8 (lw + NL i) .. + 7: lane -> row + lane / 8,
    // LDS chunk lane % 8, which holds activation chunk (lane % 8) ^ swz8(row); its value-block
    // load j is the 1 KB part (c % CPS) of slot c / CPS, c = lw + NL j. (Offsets are recomputed at
    // every issue, so that no registers stay reserved for them next to the accumulators.)
    // (the panel's column offset rides in the range-checked voffset too: a last half panel then
    // reads zeros past the end of the buffer instead of bytes beyond it)
    auto xoff = [&](int i, uint32_t col_bytes) __attribute__((always_inline)) {
        const int r = (lw + NL * i) * 8 + (lane >> 3);
        return (uint32_t)r * (uint32_t)in_ld * 2u + col_bytes + (uint32_t)(((lane & 7) ^ swz8(r)) << 4);
    };
    auto woff = [&](int j) __attribute__((always_inline)) {
        const int q = (lw + NL * j) % CPS;
        if constexpr (BS == 32) {
            const int n = 16 * q + (lane >> 2);
            return (uint32_t)(n * RB + (((lane & 3) ^ swz4(n)) << 4));
        } else {
            const int n = 8 * q + (lane >> 3);
            return (uint32_t)(n * RB + (((lane & 7) ^ swz8(n)) << 4));
        }
    };

    // Sub-step records travel with the stages: the stage of sub-step s also receives the record of
    // sub-step s + D (loader 0, lanes 0..3), so that at sub-step s the record needed to issue the
    // loads of s + D is read from LDS.
    struct Rec {
        int panel, map0, map1, blk[WPL];
    };
    auto rec_from = [&](const int32_t *e) __attribute__((always_inline)) {
        Rec x;
        x.panel = __builtin_amdgcn_readfirstlane(e[0]);
        x.map0 = __builtin_amdgcn_readfirstlane(e[1 + S]);
        x.map1 = __builtin_amdgcn_readfirstlane(e[2 + S]);
        if (loader) {
#pragma unroll
            for (int j = 0; j < WPL; ++j) x.blk[j] = __builtin_amdgcn_readfirstlane(e[1 + (lw + NL * j) / CPS]);
        }
        return x;
    };
    // a loader's loads of one sub-step (record x) into stage st, and, from loader 0, the record
    // of sub-step rsidx (if valid); returns how many loads it issued
    auto issue = [&](int st, const Rec &x, int rsidx) __attribute__((always_inline)) {
        const uint32_t base = sbase + (uint32_t)st * STAGE;
        const uint32_t pcol = (uint32_t)x.panel * 128u;
#pragma unroll
        for (int i = 0; i < XPL; ++i) dma16(ra, base + (uint32_t)(lw + NL * i) * 1024u, xoff(i, pcol), 0);
        int n = XPL;
#pragma unroll
        for (int j = 0; j < WPL; ++j) {
            const int c = lw + NL * j;
            if (x.blk[j] >= 0) {
                const uint32_t dst = base + XB + (uint32_t)(c / CPS) * WBB + (uint32_t)(c % CPS) * 1024u;
                if constexpr (SP == kCompact24) {
                    const int q = c % CPS;
                    if (q < CB / 1024) {
                        dma16(rv, dst, (uint32_t)lane * 16u, (uint32_t)x.blk[j] * CB + (uint32_t)q * 1024u);
                        ++n;
                    } else if (q == CB / 1024) {
                        dma16(rm, dst, lane < MB / 16 ? (uint32_t)lane * 16u : 0xFFFFFFF0u, (uint32_t)x.blk[j] * MB);
                        ++n;
                    }
                } else {
                    dma16(rv, dst, woff(j), (uint32_t)x.blk[j] * WBB);
                    ++n;
                }
            }
        }
        if (lw == 0 && rsidx >= 0) {
            if (lane < kRecInts / 4) dma16(rr, base + XB + S * WBB, (uint32_t)lane * 16u, (uint32_t)rsidx * kRecInts * 4u);
            ++n;
        }
        return n;
    };

    f32x16 acc[RW][GW][NT];   // [row tile][member of the wave][output tile]
#pragma unroll
    for (int rt = 0; rt < RW; ++rt)
#pragma unroll
        for (int t = 0; t < GW; ++t)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[rt][t][nt][v] = 0.f;

    // fragment of value block wb for output tile nt and 16-deep chunk kc: natural layout for the
    // forward; for the input gradient lane l holds V[kc*16 + 8 (l / 32) .. + 7][nt*32 + l % 32], from
    // two transposing reads of 4 rows each (lane s of a 16-lane group points at row R + s / 4,
    // columns C .. C + 3)
    auto wfrag = [&](const unsigned char *wb, int nt, int kc) __attribute__((always_inline)) {
        if constexpr (!TRANS) {
            const int n = nt * 32 + l32, kg = 2 * kc + lh;
            const int sw = BS == 32 ? swz4(n) : swz8(n);
            return *reinterpret_cast<const bf16x8 *>(wb + n * RB + ((kg ^ sw) << 4));
        } else {
            const int gq = lane >> 4, s16 = lane & 15;
            const int R = kc * 16 + (gq >> 1) * 8 + (s16 >> 2);
            const int C = nt * 32 + (gq & 1) * 16 + 4 * (s16 & 3);
            auto at = [&](int row) {
                const int sw = BS == 32 ? swz4(row) : swz8(row);
                return (lds_i16x4 *)(wb + row * RB + ((((C >> 3) ^ sw) << 4) | ((C & 7) << 1)));
            };
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(at(R));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(at(R + 4));
            const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            return __builtin_bit_cast(bf16x8, v);
        }
    };
    // activation fragment of 16-column chunk c of the panel (row tile rt of the wave: 32 rows)
    auto xfrag = [&](const unsigned char *xt, int rt, int c) __attribute__((always_inline)) {
        const int r = (wr * RW + rt) * 32 + l32;
        return *reinterpret_cast<const bf16x8 *>(xt + r * 128 + (((2 * c + lh) ^ swz8(r)) << 4));
    };
    auto slot_of = [&](int u, int map0, int map1) __attribute__((always_inline)) {
        return ((u < 8 ? map0 : map1) >> (4 * (u % 8))) & 15;
    };

    // Products of one staged sub-step, panel half by panel half: the wave's activation fragments of
    // the half, then for every member of the wave with a block there (uniform tests) its value
    // fragments and products. (Reading every unit's fragments first, absent ones included, and
    // skipping only the products measured slower: the extra LDS reads slow the loads landing in LDS.)
    auto compute = [&](int st, int map0, int map1) __attribute__((always_inline)) {
        const unsigned char *xt = smem + st * STAGE;
        const unsigned char *wt = xt + XB;
#pragma unroll
        for (int h = 0; h < PB; ++h) {
            bf16x8 xf[RW][KCB];
#pragma unroll
            for (int rt = 0; rt < RW; ++rt)
#pragma unroll
                for (int kc = 0; kc < KCB; ++kc) xf[rt][kc] = xfrag(xt, rt, h * KCB + kc);
#pragma unroll
            for (int t = 0; t < GW; ++t) {
                const int slot = slot_of((wm * GW + t) * PB + h, map0, map1);
                if (slot == 15) continue;
                const unsigned char *wb = wt + slot * WBB;
                if constexpr (SP == kCompact24) {
                    // compressed block: lane (n, half lh) takes the 8 kept values of columns 32 kk +
                    // 16 lh .. + 15 of row n and their index word (as with the image below)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        const int n = nt * 32 + l32;
#pragma unroll
                        for (int kk = 0; kk < KCB / 2; ++kk) {
                            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(wb + n * BS + (2 * kk + lh) * 16);
                            const int idx = (int)*reinterpret_cast<const uint16_t *>(wb + CB + n * (BS / 8) + (2 * kk + lh) * 2);
#pragma unroll
                            for (int rt = 0; rt < RW; ++rt) {
                                const bf16x16 bx = __builtin_shufflevector(xf[rt][2 * kk], xf[rt][2 * kk + 1], 0, 1, 2, 3,
                                                                           4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
                                acc[rt][t][nt] =
                                    __builtin_amdgcn_smfmac_f32_32x32x32_bf16(a, bx, acc[rt][t][nt], idx, 0, 0);
                            }
                        }
                    }
                    continue;
                }
                if constexpr (SP == kImage24) {
                    // 2:4 image of the block: row n holds the row's kept values in 16-byte chunks
                    // 0 .. BS/16 - 1 and its 16-bit index words at the start of chunk BS/16 (the
                    // loaders stage it like a bf16 block of the same size). One sparse MFMA per
                    // 32 columns: lane (n, half lh) takes the kept values of columns 32 kk + 16 lh ..
                    // + 15 and their 16 index bits; the activation operand is the two 16-deep
                    // fragments of those 32 columns, concatenated.
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        const int n = nt * 32 + l32;
                        const int sw = BS == 32 ? swz4(n) : swz8(n);
                        const unsigned char *row = wb + n * RB;
#pragma unroll
                        for (int kk = 0; kk < KCB / 2; ++kk) {
                            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(row + (((2 * kk + lh) ^ sw) << 4));
                            const uint32_t mw =
                                *reinterpret_cast<const uint32_t *>(row + (((BS / 16) ^ sw) << 4) + 4 * kk);
                            const int idx = (int)((mw >> (16 * lh)) & 0xFFFFu);
#pragma unroll
                            for (int rt = 0; rt < RW; ++rt) {
                                const bf16x16 bx = __builtin_shufflevector(xf[rt][2 * kk], xf[rt][2 * kk + 1], 0, 1, 2, 3,
                                                                           4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
                                acc[rt][t][nt] =
                                    __builtin_amdgcn_smfmac_f32_32x32x32_bf16(a, bx, acc[rt][t][nt], idx, 0, 0);
                            }
                        }
                    }
                    continue;
                }
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    bf16x8 wf[KCB];
#pragma unroll
                    for (int kc = 0; kc < KCB; ++kc) wf[kc] = wfrag(wb, nt, kc);
#pragma unroll
                    for (int kc = 0; kc < KCB; ++kc)
#pragma unroll
                        for (int rt = 0; rt < RW; ++rt)
                            acc[rt][t][nt] = mfma32(wf[kc], xf[rt][kc], acc[rt][t][nt]);
                }
            }
        }
    };

    const int s0 = sub_ptr[g], s1 = sub_ptr[g + 1];
    if (s0 < s1) {
        // Stage q holds sub-step q's panel and value blocks and the record of sub-step q + D. The
        // prologue puts sub-steps s0 .. s0 + D - 1 in flight.
        int mp0[D], mp1[D];   // unit maps of sub-steps s .. s + D - 1
        int nlast = 0;        // loads this loader issued for the latest sub-step in flight
#pragma unroll
        for (int q = 0; q < D; ++q) {
            mp0[q] = mp1[q] = -1;
            if (s0 + q < s1) {
                const Rec x = rec_from(rec + (size_t)(s0 + q) * kRecInts);
                if (loader) nlast = issue(q, x, s0 + q + D < s1 ? s0 + q + D : -1);
                mp0[q] = x.map0;
                mp1[q] = x.map1;
            }
        }
        int st = 0;   // stage of sub-step s
        for (int s = s0; s < s1; ++s) {
            // this loader's loads of sub-step s have landed (those of s + 1 .. s + D - 1 may not)
            if (loader) {
                if (D == 2 && s + 1 < s1) wait_vm<0, MAXL>(nlast);
                else wait_vm<0, 0>(0);
            }
            __syncthreads();   // everyone's have; nobody reads sub-step s - 1 any more
            int m0 = -1, m1 = -1;
            if (s + D < s1) {
                const Rec x = rec_from(reinterpret_cast<const int32_t *>(smem + st * STAGE + XB + S * WBB));
                // into the stage of s - 1
                if (loader) nlast = issue(st == 0 ? NST - 1 : st - 1, x, s + 2 * D < s1 ? s + 2 * D : -1);
                m0 = x.map0;
                m1 = x.map1;
            } else {
                nlast = 0;
            }
            if (!loader) compute(st, mp0[0], mp1[0]);
#pragma unroll
            for (int q = 0; q + 1 < D; ++q) {
                mp0[q] = mp0[q + 1];
                mp1[q] = mp1[q + 1];
            }
            mp0[D - 1] = m0;
            mp1[D - 1] = m1;
            st = st == NST - 1 ? 0 : st + 1;
        }
    }
    // Epilogue, through LDS: the compute waves write their rows x members (bias added, bf16) into the
    // staged tile of BM rows x G*BS columns, then each stores 32 rows as 16-byte pieces, 64 lanes
    // covering whole 64-byte block rows (instead of 8-byte pieces spread over 32 rows). With MS > 1
    // a stored row holds columns of several waves: a barrier separates the two phases.
    __syncthreads();   // every wave is done with the stages
    constexpr int OC = G * BS;              // output columns of the work-group
    constexpr int OP = OC * 2 + 16;         // LDS pitch of a staged output row (bytes)
    static_assert(NW * 32 * OP <= NST * STAGE, "output staging fits in the stages");
    if (!loader) {
        // item v of lane l is output column nt*32 + 8*(v/4) + 4*(l/32) + v%4 of member t, row l%32
#pragma unroll
        for (int t = 0; t < GW; ++t) {
            const int tg = wm * GW + t;
            const int o = gout[g * G + tg];
            if (o < 0) continue;
#pragma unroll
            for (int rt = 0; rt < RW; ++rt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int c = tg * BS + nt * 32 + q * 8 + lh * 4;
                        const int row = (wr * RW + rt) * 32 + l32;
                        f32x4 v = quad(acc[rt][t][nt], q);
                        if (bias) v = add_bias4(v, bias + o * BS + nt * 32 + q * 8 + lh * 4);
                        store4_bf16(reinterpret_cast<uint16_t *>(smem + row * OP + c * 2), v[0], v[1], v[2], v[3]);
                    }
        }
    }
    if constexpr (MS > 1) __syncthreads();   // the staged tile is complete
    if (loader) return;
    const unsigned char *ot = smem + wave * 32 * OP;
    const int m0 = mt0 * BM + wave * 32;
    constexpr int SPR = OC / 8;             // 16-byte pieces per row
#pragma unroll
    for (int i = 0; i < 32 * SPR / 64; ++i) {
        const int seg = i * 64 + lane, row = seg / SPR, cs = seg % SPR;
        const int t = cs * 8 / BS, within = cs * 8 % BS;
        const int o = gout[g * G + t];
        if (o < 0 || m0 + row >= M) continue;
        const u32x4 val = *reinterpret_cast<const u32x4 *>(ot + row * OP + cs * 16);
        // streaming (nontemporal) store: the output is written once and not read back here, so it
        // should not push the activation panels and value blocks out of L2 and the last-level cache
        // (BERT-base FFN-up forward 28.8 -> 22.7 us)
        __builtin_nontemporal_store(val, reinterpret_cast<u32x4 *>(out + (int64_t)(m0 + row) * out_ld + o * BS + within));
    }
}

// ------------------------------------------------------------------------------------------
// Small-M forward (M <= 64, MT tiles of 16 rows per grid row y): a streaming pass over the block values, the memory-bound regime
// where the kept blocks are loaded once and expanded into dense matrix-core products (GPU MODE
// lecture 11 summary, 48:12, "load and sparse expand"). Work-group = PSW consecutive 16-row slices
// of one block row (rows are dealt heaviest first); its NW waves take the row's kept blocks U at a
// time (wave w: blocks w*U .. w*U + U - 1 of each pass of NW*U), each reading its slices of whole
// blocks (PSW*16 rows: contiguous bytes) and the activation columns of each block once for all
// its slices. Every load of a pass is requested before the first product. The waves' partial
// products are summed in LDS in wave order (deterministic).
//   slice s:  A[p][k] = V[i][s*16 + p][k]   B[k][m] = X[m][c*BS + k]   (m < 16; rows past M are 0)
// ------------------------------------------------------------------------------------------
// ROWPTR: `rows` is a CSR row pointer (block row r = work-group / PARTS, blocks row_ptr[r] ..
// row_ptr[r+1]) instead of the host-built list; used with metadata rebuilt on the device. Block
// positions are clamped to `cap` (the blocks col_idx and V hold), so a row pointer whose total
// exceeds them never reads past either array.
// WORK: `rows` is the balanced work list, one entry per work-group {row, first, end, first slice |
// slices << 8} with 1 or 2 slices (PSW = 2).
template <int BS, int NW, int U, int PSW, bool PIPE = false, bool ROWPTR = false, bool WORK = false, int MT = 1>
__global__ __launch_bounds__(NW * 64) void k_small_m(const uint16_t *__restrict__ X, int K, int M,
                                                     const uint16_t *__restrict__ V, const uint16_t *__restrict__ bias,
                                                     uint16_t *__restrict__ Y, int N, const int32_t *__restrict__ col_idx,
                                                     const int32_t *__restrict__ rows, int cap = 0) {
    constexpr int PS = PSW;       // 16-row slices of each block handled by this work-group
    constexpr int KC = BS / 32;   // 32-deep k chunks per block
    constexpr int PARTS = BS / 16 / PSW;
    __shared__ f32x4 red[NW][MT * PS][64];

    // work-group entry {block row, first block, end block}: one read ahead of the first value loads
    int4 e;
    if constexpr (ROWPTR) {
        const int rr = (int)(blockIdx.x / PARTS);
        e = int4{rr, min(rows[rr], cap), min(rows[rr + 1], cap), 0};
    } else if constexpr (WORK) {
        e = reinterpret_cast<const int4 *>(rows)[blockIdx.x];
    } else {
        e = reinterpret_cast<const int4 *>(rows)[blockIdx.x / PARTS];
    }
    const int r = e.x, i1 = e.z;
    const int s0 = WORK ? (e.w & 0xff) : (int)(blockIdx.x % PARTS) * PSW;   // first slice
    const int ns = WORK ? (e.w >> 8) : PS;                                  // slices (uniform)
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int l16 = lane & 15, lq = lane >> 4;
    // this work-group's MT tiles of 16 activation rows, m0 .. m0 + 16 MT - 1 (grid row y); rows past M
    // read as zero. Each value fragment feeds the products of all MT tiles.
    const int m0 = blockIdx.y * 16 * MT, Mc = min(16 * MT, M - m0);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(X + (int64_t)m0 * K, (uint32_t)Mc * K * 2);
    const uint32_t xoff = (uint32_t)(l16 * K + lq * 8) * 2;
    const uint32_t xend = (uint32_t)Mc * K * 2;   // past this chunk's activations: reads zeros
    const uint32_t voff = (uint32_t)((s0 * 16 + l16) * BS + lq * 8) * 2;   // + s * 16 rows + kc * 32 columns

    f32x4 acc[MT][PS];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int s = 0; s < PS; ++s) acc[t][s] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the loads of one pass (this wave's blocks ib .. ib + U - 1): the value loads need only the
    // block index, so they are requested before the column indices, whose read would otherwise delay
    // them
    auto load_pass = [&](int ib, bf16x8 (&a)[U][PS][KC], bf16x8 (&b)[U][MT][KC]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int iu = ib + u;
            const __amdgpu_buffer_rsrc_t rv =
                make_rsrc(V + (size_t)min(iu, i1 - 1) * BS * BS, iu < i1 ? BS * BS * 2 : 0);
#pragma unroll
            for (int s = 0; s < PS; ++s)
                if (s < ns) {
#pragma unroll
                    for (int kc = 0; kc < KC; ++kc) a[u][s][kc] = buf_load16(rv, voff + (s * 16 * BS + kc * 32) * 2, 0);
                }
        }
        int col[U];
#pragma unroll
        for (int u = 0; u < U; ++u) col[u] = col_idx[min(ib + u, i1 - 1)];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // blocks past the row's end read zeros for both operands (a zero block times a
            // non-finite activation would not be zero). The block column rides in the
            // range-checked voffset, so no column index makes the load leave the activations.
            const uint32_t xo = ib + u < i1 ? xoff : xend;
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int kc = 0; kc < KC; ++kc)
                    b[u][t][kc] = buf_load16(rx, xo + (uint32_t)t * 16u * (uint32_t)K * 2u + kc * 64 + (uint32_t)col[u] * BS * 2, 0);
        }
    };
    auto compute_pass = [&](const bf16x8 (&a)[U][PS][KC], const bf16x8 (&b)[U][MT][KC]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int s = 0; s < PS; ++s)
                if (s < ns) {
#pragma unroll
                    for (int t = 0; t < MT; ++t)
#pragma unroll
                        for (int kc = 0; kc < KC; ++kc) acc[t][s] = mfma(a[u][s][kc], b[u][t][kc], acc[t][s]);
                }
    };
    if constexpr (!PIPE) {
        for (int i0 = e.y; i0 < i1; i0 += NW * U) {
            bf16x8 a[U][PS][KC], b[U][MT][KC];
            load_pass(i0 + wave * U, a, b);
            __builtin_amdgcn_sched_barrier(0);   // keep the products after every load
            compute_pass(a, b);
        }
    } else {
        // two register sets: the loads of the next pass are requested before the products of the
        // current one, so a row's passes overlap their memory latency instead of chaining it
        bf16x8 aA[U][PS][KC], bA[U][MT][KC], aB[U][PS][KC], bB[U][MT][KC];
        int i0 = e.y;
        if (i0 < i1) load_pass(i0 + wave * U, aA, bA);
        while (i0 < i1) {
            const int n1 = i0 + NW * U;
            if (n1 < i1) load_pass(n1 + wave * U, aB, bB);
            __builtin_amdgcn_sched_barrier(0);
            compute_pass(aA, bA);
            if (n1 >= i1) break;
            const int n2 = n1 + NW * U;
            if (n2 < i1) load_pass(n2 + wave * U, aA, bA);
            __builtin_amdgcn_sched_barrier(0);
            compute_pass(aB, bB);
            i0 = n2;
        }
    }
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int s = 0; s < PS; ++s) red[wave][t * PS + s][lane] = acc[t][s];
    __syncthreads();
    // wave w < PS sums slice w over the waves; lane l holds output rows n = 4 (l / 16) .. + 3 of the
    // slice for activation row l % 16
    if (wave < ns) {
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            f32x4 v = red[0][t * PS + wave][lane];
#pragma unroll
            for (int w = 1; w < NW; ++w) v += red[w][t * PS + wave][lane];
            const int row = t * 16 + l16;
            if (row < Mc) {
                const int n = r * BS + (s0 + wave) * 16 + lq * 4;
                if (bias) v = add_bias4(v, bias + n);
                store4_bf16(Y + (int64_t)(m0 + row) * N + n, v[0], v[1], v[2], v[3]);
            }
        }
    }
}

// ------------------------------------------------------------------------------------------
// Small-M forward over the balanced work list, with the value slices loaded as whole cache lines.
// Same work split, products and reduction as k_small_m (WORK, one block per wave and pass, the
// next pass's loads requested before the current pass's products), but each value load reads 1 KB
// contiguous (8 rows x 128 bytes for b = 64, 16 rows x 64 bytes for b = 32) into registers, and
// the wave re-lays it through its own 4 KB of LDS (16-byte chunks XOR-swizzled per row) into the
// matrix-core fragments (row l % 16, chunk 4 kc + l / 16). Loading the fragments straight from
// memory puts 16 rows x 64 bytes (16 half lines) in every load: a plain streaming probe on one
// MI355X reads a 64 MB set in 13.4 us that way against 9.2 us with 1 KB contiguous per load. Every
// load is an ordinary one, so the compiler's waits are exact; no barrier inside the loop (a wave
// reads back only its own writes).
// ------------------------------------------------------------------------------------------
template <int BS>
__device__ __forceinline__ int vswz(int r) {
    if constexpr (BS == 64) return swz8(r);
    else return swz4(r);
}

template <int BS, int NW, int MT, int NB>
__global__ __launch_bounds__(NW * 64) void k_small_m_lines(const uint16_t *__restrict__ X, int K, int M,
                                                           const uint16_t *__restrict__ V,
                                                           const uint16_t *__restrict__ bias, uint16_t *__restrict__ Y,
                                                           int N, const int32_t *__restrict__ col_idx,
                                                           const int32_t *__restrict__ work) {
    constexpr int PS = 2, KC = BS / 32;
    constexpr int RB = BS * 2;             // bytes of one block row
    constexpr int SLB = 16 * RB;           // one 16-row slice of a block (2 KB for b = 64, 1 KB for 32)
    constexpr int DPS = SLB / 1024;        // 1 KB loads per slice (= KC)
    constexpr int LPR = RB / 16;           // lanes per block row in a load
    constexpr int RPL = 64 / LPR;          // block rows per load
    constexpr int WB = PS * SLB;           // a wave's LDS region (both slices of one block)
    constexpr int RED = NW * MT * PS * 64 * 16;
    static_assert(DPS == KC, "one 1 KB load per 32-deep chunk of a slice");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[NW * WB > RED ? NW * WB : RED];

    const int4 e = reinterpret_cast<const int4 *>(work)[blockIdx.x];
    const int r = e.x, i1 = e.z;
    const int s0 = e.w & 0xff, ns = e.w >> 8;   // first slice, slices (1 or 2; uniform)
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int l16 = lane & 15, lq = lane >> 4;
    const int m0 = blockIdx.y * 16 * MT, Mc = min(16 * MT, M - m0);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(X + (int64_t)m0 * K, (uint32_t)Mc * K * 2);
    const uint32_t xoff = (uint32_t)(l16 * K + lq * 8) * 2;
    const uint32_t xend = (uint32_t)Mc * K * 2;   // past this chunk's activations: reads zeros
    unsigned char *wreg = smem + wave * WB;

    // load d of a slice: block row d * RPL + lane / LPR, 16-byte chunk lane % LPR (source offset),
    // written to LDS at chunk (lane % LPR) ^ swizzle(row)
    const int lrow = lane / LPR, lchunk = lane % LPR;
    auto load_pass = [&](int ib, bf16x8 (&v)[PS][KC], bf16x8 (&b)[MT][KC]) __attribute__((always_inline)) {
        // blocks past the row's end read zeros for both operands (a zero block times a non-finite
        // activation would not be zero)
        const bool in = ib < i1;
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + (size_t)min(ib, i1 - 1) * BS * BS, in ? BS * BS * 2 : 0);
#pragma unroll
        for (int sl = 0; sl < PS; ++sl)
            if (sl < ns) {
#pragma unroll
                for (int d = 0; d < DPS; ++d)
                    v[sl][d] = buf_load16(rv, (uint32_t)((s0 + sl) * SLB + (d * RPL + lrow) * RB + lchunk * 16), 0);
            }
        const int col = col_idx[min(ib, i1 - 1)];
        const uint32_t xo = in ? xoff : xend;
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
                b[t][kc] = buf_load16(rx, xo + (uint32_t)t * 16u * (uint32_t)K * 2u + kc * 64 + (uint32_t)col * BS * 2, 0);
    };

    f32x4 acc[MT][PS];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int sl = 0; sl < PS; ++sl) acc[t][sl] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute_pass = [&](const bf16x8 (&v)[PS][KC], const bf16x8 (&b)[MT][KC]) __attribute__((always_inline)) {
#pragma unroll
        for (int sl = 0; sl < PS; ++sl)
            if (sl < ns) {
#pragma unroll
                for (int d = 0; d < DPS; ++d) {
                    const int row = d * RPL + lrow;
                    *reinterpret_cast<bf16x8 *>(wreg + sl * SLB + row * RB + ((lchunk ^ vswz<BS>(row)) << 4)) = v[sl][d];
                }
            }
        bf16x8 a[PS][KC];
#pragma unroll
        for (int sl = 0; sl < PS; ++sl)
            if (sl < ns) {
#pragma unroll
                for (int kc = 0; kc < KC; ++kc)
                    a[sl][kc] = *reinterpret_cast<const bf16x8 *>(wreg + sl * SLB + l16 * RB +
                                                                 (((kc * 4 + lq) ^ vswz<BS>(l16)) << 4));
            }
#pragma unroll
        for (int sl = 0; sl < PS; ++sl)
            if (sl < ns) {
#pragma unroll
                for (int t = 0; t < MT; ++t)
#pragma unroll
                    for (int kc = 0; kc < KC; ++kc) acc[t][sl] = mfma(a[sl][kc], b[t][kc], acc[t][sl]);
            }
    };

    // this wave's blocks: e.y + wave, + NW, ...; NB register sets in a ring, the loads of the pass
    // NB - 1 ahead requested before the current pass's products
    bf16x8 vs[NB][PS][KC], bs[NB][MT][KC];
    const int ib0 = e.y + wave;
#pragma unroll
    for (int q = 0; q < NB - 1; ++q)
        if (ib0 + q * NW < i1) load_pass(ib0 + q * NW, vs[q], bs[q]);
    for (int ib = ib0; ib < i1;) {
#pragma unroll
        for (int q = 0; q < NB; ++q) {
            const int ahead = ib + (NB - 1) * NW;
            if (ahead < i1) load_pass(ahead, vs[(q + NB - 1) % NB], bs[(q + NB - 1) % NB]);
            __builtin_amdgcn_sched_barrier(0);
            compute_pass(vs[q], bs[q]);
            ib += NW;
            if (ib >= i1) break;
        }
    }
    __syncthreads();   // every wave's region is free for the reduction
    f32x4 (*red)[MT * PS][64] = reinterpret_cast<f32x4 (*)[MT * PS][64]>(smem);
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int sl = 0; sl < PS; ++sl) red[wave][t * PS + sl][lane] = acc[t][sl];
    __syncthreads();
    // wave w < ns sums slice w over the waves; lane l holds output rows n = 4 (l / 16) .. + 3 of the
    // slice for activation row l % 16
    if (wave < ns) {
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            f32x4 v = red[0][t * PS + wave][lane];
#pragma unroll
            for (int w = 1; w < NW; ++w) v += red[w][t * PS + wave][lane];
            const int row = t * 16 + l16;
            if (row < Mc) {
                const int n = r * BS + (s0 + wave) * 16 + lq * 4;
                if (bias) v = add_bias4(v, bias + n);
                store4_bf16(Y + (int64_t)(m0 + row) * N + n, v[0], v[1], v[2], v[3]);
            }
        }
    }
}

// ------------------------------------------------------------------------------------------
// Weight gradient on the kept blocks (block-masked SDDMM): for block i of row r, column c,
//   dV[i][p][q] = sum_m dY[m][r*BS + p] * X[m][c*BS + q].
// Work-group = (item, chunk of M); an item is up to kDwWaves * SL kept blocks of one tile of TR
// consecutive block rows by TC consecutive block columns (see DwSchedule). Per stage of KM = 32
// activation rows, two loader waves stage the tile's dY row segments (TR * BS columns, 512 bytes)
// and X row segments (TC * BS columns, 1 KB) into LDS with direct-to-LDS loads, three stages
// deep; every compute wave then runs the products of its blocks from transposing LDS reads:
//   D[p][q] += A[p][k] . B[k][q],   A[p][k] = dY[m0 + k][r*BS + p],   B[k][q] = X[m0 + k][c*BS + q]
// (32x32x16 MFMA; lane l ends up with rows 8 (v / 4) + 4 (l / 32) + v % 4 of column l % 32).
// The 16-byte chunks of each staged row are XOR swizzled by 4 * (row % 4), which keeps the
// transposing reads (4 rows x 2 chunks per 16 lanes) free of bank conflicts. With one chunk of M
// the sums are rounded to bf16 directly; otherwise fp32 partials [chunk][block] go to the
// workspace for k_dw_reduce.
// ------------------------------------------------------------------------------------------
template <int BS, int NL>
__global__ __launch_bounds__((kDwWaves + NL) * 64) void k_dw_panel(
    const uint16_t *__restrict__ dY, int N, const uint16_t *__restrict__ X, int K, int M,
    const int32_t *__restrict__ items, int nitems, const int32_t *__restrict__ live, int mchunk,
    float *__restrict__ partial, int nnzb, uint16_t *__restrict__ dV) {
    constexpr int NW = kDwWaves;
    constexpr int SL = BS == 64 ? 2 : 8;        // blocks per compute wave (dw_slots)
    constexpr int NT = BS / 32;                 // 32 x 32 sub-tiles per block side
    constexpr int KM = 32;                      // activation rows per stage
    constexpr int DB = 512, XR = 1024;          // bytes per staged row: dY segment, X segment
    constexpr int DS = KM * DB, XS = KM * XR;
    constexpr int STAGE = DS + XS;
    constexpr int NST = 3;
    constexpr int DPL = KM / 2 / NL;            // dY loads (2 rows each) per loader wave and stage
    constexpr int XPL = KM / NL;                // X loads (1 row each) per loader wave and stage
    constexpr int NLD = DPL + XPL;
    static_assert(KM / 2 % NL == 0 && KM % NL == 0 && 2 * NLD <= 63, "loader split");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[NST * STAGE];

    // each XCD takes a contiguous run of (chunk, item) pairs, items fastest
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int item = L % nitems, ch = L / nitems;
    if (live && item >= *live) return;   // a device-built list shorter than its capacity
    const int32_t *it = items + (size_t)item * kDwItemInts;
    const int r0 = it[0], c0 = it[1];
    const int m_begin = ch * mchunk, m_end = min(M, m_begin + mchunk);
    const int nst = (m_end - m_begin + KM - 1) / KM;   // mchunk is a multiple of KM
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool loader = wave >= NW;
    const int lw = wave - NW;
    const int l32 = lane & 31, lh = lane >> 5;
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(dY, (uint32_t)((size_t)M * N * 2));
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(X, (uint32_t)((size_t)M * K * 2));
    const uint32_t sbase = lds_addr(smem);

    // loads of one stage (activation rows m0 .. m0 + KM - 1) into stage st: staged chunk c of row
    // `row` holds source chunk c ^ 4 (row % 4). Offsets stay in the range-checked voffset, so rows
    // past M and columns past the matrix end read as zeros.
    auto issue = [&](int st, int m0) __attribute__((always_inline)) {
        const uint32_t base = sbase + (uint32_t)st * STAGE;
#pragma unroll
        for (int d = 0; d < DPL; ++d) {
            const int ins = lw + NL * d, row = 2 * ins + (lane >> 5);
            const uint32_t voff = (uint32_t)(m0 + row) * (uint32_t)N * 2u + (uint32_t)r0 * BS * 2u +
                                  (uint32_t)(((lane & 31) ^ ((row & 3) << 2)) << 4);
            dma16(rd, base + (uint32_t)ins * 1024u, voff, 0);
        }
#pragma unroll
        for (int x = 0; x < XPL; ++x) {
            const int row = lw + NL * x;
            const uint32_t voff = (uint32_t)(m0 + row) * (uint32_t)K * 2u + (uint32_t)c0 * BS * 2u +
                                  (uint32_t)((lane ^ ((row & 3) << 2)) << 4);
            dma16(rx, base + DS + (uint32_t)row * 1024u, voff, 0);
        }
    };

    // T[k0 + 8 (l / 32) .. + 7][n0 + l % 32] of a staged tile (rows of `pitch` bytes), for lane l:
    // two transposing reads of 4 rows; lane s of a 16-lane group points at row R + s / 4, columns
    // C .. C + 3 (8 bytes inside one 16-byte chunk)
    auto frag = [&](const unsigned char *t, int pitch, int k0, int n0) __attribute__((always_inline)) {
        const int gq = lane >> 4, s16 = lane & 15;
        const int R = k0 + (gq >> 1) * 8 + (s16 >> 2);
        const int C = n0 + (gq & 1) * 16 + 4 * (s16 & 3);
        auto at = [&](int row) {
            return (lds_i16x4 *)(t + row * pitch + ((((C >> 3) ^ ((row & 3) << 2)) << 4) | ((C & 7) << 1)));
        };
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(at(R));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(at(R + 4));
        const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return __builtin_bit_cast(bf16x8, v);
    };

    int nq = 0, word[SL];
    if (!loader) {
        nq = it[2 + wave];
#pragma unroll
        for (int q = 0; q < SL; ++q) word[q] = it[16 + 8 * wave + q];
    }
    f32x16 acc[SL][NT][NT];
#pragma unroll
    for (int q = 0; q < SL; ++q)
#pragma unroll
        for (int pt = 0; pt < NT; ++pt)
#pragma unroll
            for (int qt = 0; qt < NT; ++qt)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[q][pt][qt][v] = 0.f;

    auto compute = [&](int st) __attribute__((always_inline)) {
        const unsigned char *dt = smem + st * STAGE, *xt = dt + DS;
#pragma unroll
        for (int q = 0; q < SL; ++q) {
            if (q >= nq) break;
            const int i = (word[q] >> 4) & 15, j = word[q] & 15;
#pragma unroll
            for (int kc = 0; kc < KM / 16; ++kc) {
                bf16x8 a[NT], bq[NT];
#pragma unroll
                for (int pt = 0; pt < NT; ++pt) a[pt] = frag(dt, DB, kc * 16, i * BS + pt * 32);
#pragma unroll
                for (int qt = 0; qt < NT; ++qt) bq[qt] = frag(xt, XR, kc * 16, j * BS + qt * 32);
#pragma unroll
                for (int pt = 0; pt < NT; ++pt)
#pragma unroll
                    for (int qt = 0; qt < NT; ++qt) acc[q][pt][qt] = mfma32(a[pt], bq[qt], acc[q][pt][qt]);
            }
        }
    };

    if (loader) {
        issue(0, m_begin);
        if (nst > 1) issue(1, m_begin + KM);
    }
    int st = 0;
    for (int s = 0; s < nst; ++s) {
        if (loader) {
            if (s + 1 < nst) wait_vm<NLD, NLD>(NLD);   // this loader's loads of stage s have landed
            else wait_vm<0, 0>(0);
        }
        __syncthreads();   // everyone's have; nobody reads the stage of s - 1 any more
        if (loader && s + 2 < nst) issue(st == 0 ? 2 : st - 1, m_begin + (s + 2) * KM);
        if (!loader) compute(st);
        st = st == 2 ? 0 : st + 1;
    }
    if (loader) return;

    // item v of lane l: row pt*32 + 8 (v / 4) + 4 (l / 32) + v % 4, column qt*32 + l % 32
#pragma unroll
    for (int q = 0; q < SL; ++q) {
        if (q >= nq) break;
        const int blk = word[q] >> 8;
#pragma unroll
        for (int pt = 0; pt < NT; ++pt)
#pragma unroll
            for (int qt = 0; qt < NT; ++qt)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int pp = pt * 32 + 8 * (v / 4) + 4 * lh + v % 4, qq = qt * 32 + l32;
                    const size_t e = (size_t)pp * BS + qq;
                    if (partial) partial[((size_t)ch * nnzb + blk) * BS * BS + e] = acc[q][pt][qt][v];
                    else dV[(size_t)blk * BS * BS + e] = to_bf16(acc[q][pt][qt][v]);
                }
    }
}

// dV[b][e] = bf16(sum over chunks of partial[chunk][b][e]), 4 elements per thread. The partials are
// read once: streaming (nontemporal) loads keep them from displacing cached activations (square
// 8192 x 4096 -> 4096 at density 0.1, weight gradients launched back to back: 101.6 -> 94.5 us; no
// change inside a full training step. Issuing 8 chunks' loads before their sums was slower on
// BERT-base FFN-up, 25.0 -> 26.4 us).
__global__ __launch_bounds__(256) void k_dw_reduce(const float *__restrict__ partial, int nchunks, size_t count,
                                                   uint16_t *__restrict__ dV) {
    const size_t e = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (e >= count) return;
    f32x4 s = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(partial + e));
    for (int ch = 1; ch < nchunks; ++ch)
        s += __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(partial + (size_t)ch * count + e));
    store4_bf16(dV + e, s[0], s[1], s[2], s[3]);
}

// Bias gradient, pass 1: fp32 column sums of dY over one chunk of rows. Work-group = 64 columns x one
// chunk; thread t takes row lane t / 8 (rows m0 + lane, + 32, ...) and the 8 columns 8 (t % 8) ..,
// so 8 threads read one row's 128-byte segment with 16-byte loads. A thread issues the loads of 8
// of its rows before adding them in row order; the 32 row lanes are then added in lane order through
// LDS. (A thread per column reading 2 bytes per row, one row at a time, took 66 us beside a 25 us
// weight gradient on BERT-base FFN-up.)
__global__ __launch_bounds__(256) void k_colsum_partial(const uint16_t *__restrict__ dY, int N, int64_t M,
                                                        int64_t rows_per, float *__restrict__ partial) {
    constexpr int RL = 32, U = 8;
    __shared__ float red[RL][64];
    const int t = threadIdx.x, lr = t >> 3, piece = t & 7;
    const int n0 = blockIdx.x * 64 + piece * 8;
    const int64_t m0 = (int64_t)blockIdx.y * rows_per, m1 = std::min<int64_t>(M, m0 + rows_per);
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (n0 < N) {   // N is a multiple of 32: a thread's 8 columns are all inside or all outside
        for (int64_t mb = m0 + lr; mb < m1; mb += (int64_t)RL * U) {
            u32x4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t m = mb + (int64_t)RL * u;
                v[u] = m < m1 ? *reinterpret_cast<const u32x4 *>(dY + m * N + n0) : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (mb + (int64_t)RL * u >= m1) break;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    s[2 * j] += from_bf16((uint16_t)(v[u][j] & 0xffffu));
                    s[2 * j + 1] += from_bf16((uint16_t)(v[u][j] >> 16));
                }
            }
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) red[lr][piece * 8 + j] = s[j];
    __syncthreads();
    const int n = blockIdx.x * 64 + t;
    if (t < 64 && n < N) {
        float c = red[0][t];
        for (int l = 1; l < RL; ++l) c += red[l][t];
        partial[(size_t)blockIdx.y * N + n] = c;
    }
}

// Bias gradient, pass 2: sum the partials in chunk order (the loads of 8 chunks issued together).
__global__ __launch_bounds__(256) void k_colsum_final(const float *__restrict__ partial, int nchunks, int N,
                                                      uint16_t *__restrict__ db) {
    constexpr int U = 8;
    const int n = blockIdx.x * 256 + threadIdx.x;
    if (n >= N) return;
    float s = 0.f;
    for (int c0 = 0; c0 < nchunks; c0 += U) {
        float v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = c0 + u < nchunks ? partial[(size_t)(c0 + u) * N + n] : 0.f;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (c0 + u < nchunks) s += v[u];
    }
    db[n] = to_bf16(s);
}

__global__ __launch_bounds__(256) void k_fill_zero(uint16_t *__restrict__ p, size_t count) {
    const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (e < count) p[e] = 0;
}

// ---- host-side planning ----

// Variant of a panel GEMM call (see gemm_variant); "fills" = at least two work-groups per compute
// unit, so that one work-group's prologue and epilogue overlap another's main loop.
int choose_variant(const bsr_pattern &p, bool transposed, int64_t M) {
    if (p.device_built) return kDeviceVariant;   // the only work lists its rebuild produces
    if (const char *f = std::getenv("BSR_GEMM_VARIANT")) {   // tuning knob: 0 | 1 | 2 | 3
        const int k = std::atoi(f);
        if (k >= 0 && k < kGemmVariants) return k;
    }
    const GroupSchedule *s = transposed ? p.bwd : p.fwd;
    auto fills = [&](int k) {
        const int rows = gemm_variant(p.b, k).waves * 32;
        return (int64_t)s[k].ngroups * ((M + rows - 1) / rows) >= 2 * kCUs;
    };
    // Panels that often hold more than 4 kept blocks (dense groups) favour the 4-member groups:
    // every staged panel feeds more products. The 256-row tile when it still gives every CU two
    // work-groups, else the 128-row one. For sparser patterns, long chains of sub-steps per
    // work-group (>= 16) favour the 128-row 4-member tile with three LDS stages; short ones the
    // 2-member tile, three work-groups per CU, whose prologues and epilogues overlap more (measured:
    // square 8192 x 4096 -> 4096 at density 0.1, ~36 sub-steps: 88 vs 96 us; BERT-base FFN-up,
    // ~11 sub-steps: 19 vs 21 us forward).
    const int64_t nsub1 = s[1].sub_ptr.empty() ? 0 : s[1].sub_ptr.back();
    const bool splits = (double)nsub1 > 1.15 * (double)std::max<int64_t>(1, s[1].npanels);
    if (splits) return fills(0) ? 0 : fills(1) ? 1 : 2;
    const bool long_chains = nsub1 >= 16 * (int64_t)std::max(1, s[1].ngroups);
    if (long_chains && fills(1)) return 1;
    // When even the 2-member tile leaves CUs with fewer than two work-groups, single-member groups
    // double the work-groups and shorten every chain (each walks only its own block's panels), at
    // the price of staging each panel for one output block (BERT-base FFN-up input gradient, 12
    // two-member groups x 32 tiles: 24.8 -> 19.4 us; where the 2-member tile fills the chip, e.g.
    // its forward, single members are slower: 19.1 -> 24.4 us).
    return fills(2) || p.b != 32 ? 2 : 3;
}

// Weight-gradient plan: chunks of M (a multiple of the kernel's 32-row stage, at least 256 rows)
// and the workspace layout.
struct DwPlan {
    int nchunks = 1, mchunk = 0;   // tile items
    WideDwPlan wide;               // wide items (b = 32; then there are no tile items)
    size_t partial_bytes = 0;      // tile items: [nchunks][nnzb][b*b] fp32 when nchunks > 1;
                                   // wide items: [c2][P2][1024] fp32 when c2 > 1
    int bchunks = 1;               // row chunks of the bias column sums
    int64_t brows = 0;
    size_t bias_off = 0, bias_bytes = 0, total = 0;
};

DwPlan plan_dw(const bsr_pattern &p, int64_t M) {
    DwPlan d;
    if (M <= 0) return d;
    if (p.wdw.n > 0) {
        d.wide = plan_wide_dw(p, M);
        d.partial_bytes = d.wide.c2 > 1 ? (size_t)d.wide.c2 * d.wide.P2 * 1024 * sizeof(float) : 0;
    } else {
        const int64_t n = std::max(p.dw.n, 1);
        // The most chunks whose work-groups (one per compute unit at a time) still run in a single
        // round; one chunk when the items alone fill the chip. Measured on BERT-base FFN-up (24
        // items): 8 chunks 24.5 us, 10 chunks (240 work-groups) 23.3 us, 11 chunks (264: a second
        // round) 31.9 us; more chunks also cost an fp32 partial of every block each.
        const int64_t c = std::max<int64_t>(1, std::min<int64_t>(kCUs / n, M / 256));
        d.mchunk = (int)(((M + c - 1) / c + 31) / 32 * 32);
        d.nchunks = (int)((M + d.mchunk - 1) / d.mchunk);
        d.partial_bytes = d.nchunks > 1 ? (size_t)d.nchunks * p.nnzb * p.b * p.b * sizeof(float) : 0;
    }
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    d.bchunks = (int)std::min<int64_t>(64, std::max<int64_t>(1, M / 256));
    d.brows = (M + d.bchunks - 1) / d.bchunks;
    d.bchunks = (int)((M + d.brows - 1) / d.brows);
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

// Activation tiles per chunk of the work-group order (see k_panel_gemm).
int tiles_per_chunk(int nmtiles) {
    int t = 4;
    if (const char *f = std::getenv("BSR_GEMM_TPC")) t = std::atoi(f);   // tuning knob
    return std::max(1, std::min(t, nmtiles));
}

template <int BS, int G, int S, int NW, bool TRANS, int SP = kDense>
void launch_pg(const bsr_pattern &p, const GroupSchedule &s, const DevSchedule &d, const FwdArgs &a, hipStream_t st,
               const uint16_t *meta) {
    constexpr int BM = NW * 32;
    const int nmtiles = (int)((a.M + BM - 1) / BM);
    const dim3 grid((unsigned)((int64_t)s.ngroups * nmtiles));
    const uint32_t v_bytes = (uint32_t)((size_t)p.nnzb * BS * BS * (SP == kCompact24 ? 1 : 2));
    const uint32_t m_bytes = SP == kCompact24 ? (uint32_t)((size_t)p.nnzb * BS * BS / 8) : 0u;
    constexpr int NL = panel_loader_waves(NW);
    // three LDS stages (two sub-steps of loads in flight); two for the 2-member groups, which then
    // fit three work-groups per CU
    constexpr int NST = NW == 4 && G <= 2 ? 2 : 3;
    // the 256-row 4-member tile: waves of 64 rows x 2 members, each value fragment feeding two
    // products (Zipf 16384 x 4096 -> 11008: input gradient 631 -> 613 us, forward 579 -> 573 us; no
    // gain for the 128-row tiles)
    constexpr int MS = G == 4 && NW == 8 ? 2 : 1;
    hipLaunchKernelGGL((k_panel_gemm<BS, G, S, NW, NL, NST, MS, TRANS, SP>), grid, dim3((NW + NL) * 64), 0, st, a.act, a.in_ld,
                       (int)a.M, a.V, v_bytes, meta, m_bytes, a.bias, a.out, a.out_ld, d.order, d.sub_ptr, d.out, d.rec,
                       s.ngroups, nmtiles,
                       tiles_per_chunk(nmtiles));
}

// Dispatch on the block size and the variant to the instantiated kernels.
template <bool TRANS, int SP = kDense>
int32_t launch_pg_variant(const bsr_pattern &p, int k, const FwdArgs &a, hipStream_t st, const uint16_t *meta = nullptr) {
    const GroupSchedule &s = (TRANS ? p.bwd : p.fwd)[k];
    const DevSchedule &d = (TRANS ? p.dev.bwd : p.dev.fwd)[k];
    if (p.b == 32) {
        if (k == 0) launch_pg<32, 4, 8, 8, TRANS, SP>(p, s, d, a, st, meta);
        else if (k == 1) launch_pg<32, 4, 4, 4, TRANS, SP>(p, s, d, a, st, meta);
        else if (k == 2) launch_pg<32, 2, 4, 4, TRANS, SP>(p, s, d, a, st, meta);
        else launch_pg<32, 1, 2, 4, TRANS, SP>(p, s, d, a, st, meta);
    } else {
        if (k == 0) launch_pg<64, 1, 1, 8, TRANS, SP>(p, s, d, a, st, meta);
        else launch_pg<64, 1, 1, 4, TRANS, SP>(p, s, d, a, st, meta);
    }
    return BSR_OK;
}

}  // namespace

int32_t launch_group_gemm(const bsr_pattern &p, bool transposed, const FwdArgs &a, void *stream, bool sparse24,
                          const uint16_t *meta24) {
    if (!sparse24 && use_wide(p, transposed, a.M)) return launch_wide_gemm(p, transposed, a, stream);
    const hipStream_t st = (hipStream_t)stream;
    const int k = choose_variant(p, transposed, a.M);
    const GemmVariant v = gemm_variant(p.b, k);
    const GroupSchedule &s = (transposed ? p.bwd : p.fwd)[k];
    const int rows = v.waves * 32;
    const int64_t nwg = (int64_t)s.ngroups * ((a.M + rows - 1) / rows);
    if (nwg > (int64_t)INT32_MAX) return fail(BSR_ERR_INVALID_ARG, "problem too large for one launch");
    if ((size_t)p.nnzb * p.b * p.b * 2 > (size_t)UINT32_MAX)
        return fail(BSR_ERR_INVALID_ARG, "block values above 4 GiB");
    if ((int64_t)rows * a.in_ld * 2 + 256 > (int64_t)UINT32_MAX)
        return fail(BSR_ERR_INVALID_ARG, "activation rows too long for 32-bit buffer offsets");
    const int32_t rc = transposed            ? launch_pg_variant<true>(p, k, a, st)
                       : sparse24 && meta24 ? launch_pg_variant<false, kCompact24>(p, k, a, st, meta24)
                       : sparse24           ? launch_pg_variant<false, kImage24>(p, k, a, st)
                                            : launch_pg_variant<false>(p, k, a, st);
    if (rc != BSR_OK) return rc;
    return launched(transposed ? "bwd_input launch" : "fwd launch");
}

template <int BS>
void launch_small_m_rowptr(int32_t R, int32_t N, int32_t K, const int32_t *row_ptr, const int32_t *col_idx, int32_t cap,
                           const FwdArgs &a, hipStream_t st) {
    // the configurations of the host-scheduled forward, in natural row order
    constexpr int NW = 8, U = BS == 32 ? 8 : 1, PSW = 2;
    constexpr bool PIPE = BS == 64;
    const dim3 grid((unsigned)(R * (BS / 16 / PSW)), (unsigned)((a.M + 15) / 16));
    hipLaunchKernelGGL((k_small_m<BS, NW, U, PSW, PIPE, true>), grid, dim3(NW * 64), 0, st, a.act, K, (int)a.M, a.V,
                       a.bias, a.out, N, col_idx, row_ptr, cap);
}

template <int BS, int NW, int U, bool PIPE, int MT = 1>
void launch_small_m_work(const bsr_pattern &p, const FwdArgs &a, hipStream_t st) {
    const dim3 grid((unsigned)(p.small_m_work.size() / 4), (unsigned)((a.M + 16 * MT - 1) / (16 * MT)));
    hipLaunchKernelGGL((k_small_m<BS, NW, U, 2, PIPE, false, true, MT>), grid, dim3(NW * 64), 0, st, a.act, p.K,
                       (int)a.M, a.V, a.bias, a.out, p.N, p.dev.col_idx, p.dev.small_m_work);
}

template <int BS, int MT = 1, int NB = 2>
void launch_small_m_lines(const bsr_pattern &p, const FwdArgs &a, hipStream_t st) {
    const dim3 grid((unsigned)(p.small_m_work.size() / 4), (unsigned)((a.M + 16 * MT - 1) / (16 * MT)));
    hipLaunchKernelGGL((k_small_m_lines<BS, 8, MT, NB>), grid, dim3(8 * 64), 0, st, a.act, p.K, (int)a.M, a.V, a.bias,
                       a.out, p.N, p.dev.col_idx, p.dev.small_m_work);
}

template <int BS, int NW, int U, int PSW, bool PIPE>
void launch_small_m_cfg(const bsr_pattern &p, const FwdArgs &a, hipStream_t st) {
    const dim3 grid((unsigned)(p.R * (BS / 16 / PSW)), (unsigned)((a.M + 15) / 16));
    hipLaunchKernelGGL((k_small_m<BS, NW, U, PSW, PIPE>), grid, dim3(NW * 64), 0, st, a.act, p.K, (int)a.M, a.V, a.bias,
                       a.out, p.N, p.dev.col_idx, p.dev.small_m_rows);
}

int32_t launch_small_m_fwd(const bsr_pattern &p, const FwdArgs &a, void *stream) {
    const hipStream_t st = (hipStream_t)stream;
    // Default: the balanced work list (items of one or two 16-row slices, a whole number of rounds
    // of one work-group per compute unit, heavy and light items paired over the rounds) on the
    // whole-line kernel (k_small_m_lines): 8 waves x 1 block per pass, 3 passes in flight for b = 64
    // and 2 for b = 32. The same list on k_small_m (configurations 3 and 8: b = 32 8 waves x 8
    // blocks, b = 64 8 waves x 1 block with 2 passes in flight) took 13.2-13.5 us on the decode shape
    // 8 x 4096 -> 14336 (cold, HIP events) against 13.1; the row list (two slices per work-group,
    // configurations 0-5): 14.45 (8 x 1 overlapped), 14.95 (8 x 2, no overlap), 14.9 (8 x 2
    // overlapped), 15.2 (16 x 1 overlapped), 15.9 (8 x 4), 16.2 (one slice per work-group).
    int cfg = -1;
    if (const char *f = std::getenv("BSR_SMALLM_CONFIG")) cfg = std::atoi(f);   // tuning knob: 0 .. 8
    if (p.b == 32) {
        switch (cfg) {
            case 0: launch_small_m_cfg<32, 8, 8, 2, false>(p, a, st); break;
            case 1: launch_small_m_cfg<32, 8, 4, 2, true>(p, a, st); break;
            case 2: launch_small_m_cfg<32, 8, 8, 2, true>(p, a, st); break;
            case 6:
                if (a.M > 16) launch_small_m_lines<32, 2>(p, a, st);
                else launch_small_m_lines<32>(p, a, st);
                break;
            case 3:
                // rows above 16: two 16-row tiles per work-group, each value fragment loaded once
                if (a.M > 16) launch_small_m_work<32, 8, 8, false, 2>(p, a, st);
                else launch_small_m_work<32, 8, 8, false>(p, a, st);
                break;
            default:   // 6: whole-line value loads (BERT-base FFN-up weight, 8 / 16 / 32 rows: 9.3 / 7.5 /
                       // 9.4 -> 8.0 / 7.3 / 8.2 us against the 8-blocks-per-pass list kernel)
                if (a.M > 16) launch_small_m_lines<32, 2>(p, a, st);
                else launch_small_m_lines<32>(p, a, st);
                break;
        }
    } else {
        switch (cfg) {
            case 0: launch_small_m_cfg<64, 8, 2, 2, false>(p, a, st); break;
            case 1: launch_small_m_cfg<64, 8, 2, 2, true>(p, a, st); break;
            case 2: launch_small_m_cfg<64, 8, 1, 2, true>(p, a, st); break;
            case 3: launch_small_m_cfg<64, 8, 2, 1, true>(p, a, st); break;
            case 4: launch_small_m_cfg<64, 16, 1, 2, true>(p, a, st); break;
            case 5: launch_small_m_cfg<64, 8, 4, 2, false>(p, a, st); break;
            case 6:
                if (a.M > 32) launch_small_m_lines<64, 4>(p, a, st);
                else if (a.M > 16) launch_small_m_lines<64, 2>(p, a, st);
                else launch_small_m_lines<64>(p, a, st);
                break;
            case 7:
                if (a.M > 32) launch_small_m_lines<64, 4, 3>(p, a, st);
                else if (a.M > 16) launch_small_m_lines<64, 2, 3>(p, a, st);
                else launch_small_m_lines<64, 1, 3>(p, a, st);
                break;
            case 8:
                if (a.M > 32) launch_small_m_work<64, 8, 1, true, 4>(p, a, st);
                else if (a.M > 16) launch_small_m_work<64, 8, 1, true, 2>(p, a, st);
                else launch_small_m_work<64, 8, 1, true>(p, a, st);
                break;
            default:   // 7: whole-line value loads, 3 passes in flight per wave (decode shape, cold
                       // sets, three interleaved runs: 13.17-13.47 -> 13.10-13.14 us)
                if (a.M > 32) launch_small_m_lines<64, 4, 3>(p, a, st);
                else if (a.M > 16) launch_small_m_lines<64, 2, 3>(p, a, st);
                else launch_small_m_lines<64, 1, 3>(p, a, st);
                break;
        }
    }
    return launched("fwd small-M launch");
}

int32_t launch_small_m_fwd_csr(int32_t N, int32_t K, int32_t b, const int32_t *row_ptr, const int32_t *col_idx,
                               int32_t cap, const FwdArgs &a, void *stream) {
    const hipStream_t st = (hipStream_t)stream;
    if (b == 32) launch_small_m_rowptr<32>(N / b, N, K, row_ptr, col_idx, cap, a, st);
    else launch_small_m_rowptr<64>(N / b, N, K, row_ptr, col_idx, cap, a, st);
    return launched("fwd small-M (device CSR) launch");
}

size_t dw_workspace_bytes(const bsr_pattern &p, int64_t M) { return M > 0 ? plan_dw(p, M).total : 0; }

std::string kernels_of(const bsr_pattern &p, int op, int64_t M, int64_t small_max) {
    if (M <= 0) return op == 2 ? "k_fill_zero" : "";
    if (op == 3) return use_wide(p, false, M) ? "k_wide_gemm_24" : M > small_max ? "k_panel_gemm" : "k_fwd_24";
    if (p.device_built) small_max = std::min<int64_t>(small_max, kSmallM);
    if (op == 0 && M <= small_max) {
        int cfg = -1;
        if (const char *f = std::getenv("BSR_SMALLM_CONFIG")) cfg = std::atoi(f);
        // the dispatch of launch_small_m_fwd: configurations 0 .. 3 (b = 32) and 0 .. 5, 8 (b = 64)
        // run k_small_m, every other value (the default included) the whole-line kernel
        const bool classic = p.b == 32 ? (cfg >= 0 && cfg <= 3) : ((cfg >= 0 && cfg <= 5) || cfg == 8);
        const bool lines = !p.device_built && !classic;
        return lines ? "k_small_m_lines" : "k_small_m";
    }
    if (op == 0 || op == 1) return use_wide(p, op == 1, M) ? "k_wide_gemm" : "k_panel_gemm";
    if (p.nnzb == 0) return "";
    const DwPlan pl = plan_dw(p, M);
    if (p.wdw.n > 0) return pl.wide.c2 > 1 && pl.wide.P2 > 0 ? "k_wide_dw,k_wide_dw_reduce" : "k_wide_dw";
    return pl.nchunks > 1 ? "k_dw_panel,k_dw_reduce" : "k_dw_panel";
}

// ---- weight gradient without allocation: a scratch array in the code object ----
// One array per GPU, created when the library's code object is loaded on that GPU and held until
// the process ends. Its host-side name is only a stand-in: kernels get the device address that
// hipGetSymbolAddress returns for the current device, looked up once per device.
__device__ __align__(256) unsigned char scratch[BSR_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

int32_t noalloc_scratch(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return fail(BSR_ERR_HIP, "hipGetDevice failed");
    if (dev < 0 || dev >= kMaxDevices) return fail(BSR_ERR_UNSUPPORTED, "device index above 63");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(BSR_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return BSR_OK;
}

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
    // 32-bit buffer offsets: activation rows up to 256 past the rows of one call (the wide kernel's
    // surplus loads past a chunk)
    if ((size_t)(a.M + 256) * p.N * 2 > (size_t)UINT32_MAX || (size_t)(a.M + 256) * p.K * 2 > (size_t)UINT32_MAX)
        return fail(BSR_ERR_INVALID_ARG, "activations above 4 GiB for 32-bit buffer offsets");
    if (p.wdw.n > 0) {
        // every block on the wide kernel
        const int32_t rc = launch_wide_dw(p, a, pl.wide, reinterpret_cast<float *>(ws), stream);
        if (rc != BSR_OK) return rc;
    } else if (p.nnzb > 0) {
        float *partial = pl.nchunks > 1 ? reinterpret_cast<float *>(ws) : nullptr;
        const dim3 grid((unsigned)((int64_t)p.dw.n * pl.nchunks));
        constexpr int NL = kLoaderWaves, NT = (kDwWaves + NL) * 64;
        if (p.b == 32)
            hipLaunchKernelGGL((k_dw_panel<32, NL>), grid, dim3(NT), 0, st, a.dY, p.N, a.X, p.K, (int)a.M, d.dw_items,
                               p.dw.n, d.live_items, pl.mchunk, partial, p.nnzb, a.dV);
        else
            hipLaunchKernelGGL((k_dw_panel<64, NL>), grid, dim3(NT), 0, st, a.dY, p.N, a.X, p.K, (int)a.M, d.dw_items,
                               p.dw.n, d.live_items, pl.mchunk, partial, p.nnzb, a.dV);
        if (partial) {
            const size_t count = (size_t)p.nnzb * p.b * p.b;
            hipLaunchKernelGGL(k_dw_reduce, dim3((unsigned)((count / 4 + 255) / 256)), dim3(256), 0, st, partial,
                               pl.nchunks, count, a.dV);
        }
    }
    if (a.dbias) {
        float *bp = reinterpret_cast<float *>(ws + pl.bias_off);
        hipLaunchKernelGGL(k_colsum_partial, dim3((unsigned)((p.N + 63) / 64), (unsigned)pl.bchunks), dim3(256), 0,
                           st, a.dY, p.N, a.M, pl.brows, bp);
        hipLaunchKernelGGL(k_colsum_final, dim3((unsigned)((p.N + 255) / 256)), dim3(256), 0, st, bp, pl.bchunks, p.N,
                           a.dbias);
    }
    return launched("bwd_weight launch");
}

}  // namespace bsr
