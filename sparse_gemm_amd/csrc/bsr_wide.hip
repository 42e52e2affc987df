// bsr_wide.hip -- the wide-tile panel GEMM (b = 32): forward and input gradient for groups whose
// members keep blocks in most panels, the matrix-core-bound regime (e.g. block rows kept in full).
//
// Every kept block is a dense contraction on the matrix cores, zero blocks are skipped
// (pytorch_block_sparse summary page, "Technical Foundation"). What changes against the panel GEMM
// of bsr_kernels.hip is the register tile. A work-group owns 256 activation rows x kWideG = 8 output
// blocks (256 output columns) and runs 8 waves, two per SIMD: wave w owns rows [128 (w & 1), +128)
// (4 row tiles of 32) and members 2 (w >> 1), 2 (w >> 1) + 1, a 4 x 2 grid of 32 x 32 fp32
// accumulators (128 registers). While one wave of a SIMD waits (on the issue of a direct-to-LDS load,
// an LDS read or the barrier) the other issues matrix products. Per 16-deep chunk of a panel a wave
// reads 4 activation fragments and up to 2 value fragments (1 KB each) from LDS for up to 8
// products, 0.75 KB of LDS reads per product (the panel GEMM's 2 x 2 grids: 1 KB). Measured against
// one wave per SIMD with 4 x 4 grids (Zipf 16384 x 4096 -> 11008, warm): forward 534 -> 479 us,
// input gradient 551 -> 498; at density 1.0 1.27 PFLOP/s against 1.16.
//
// Sub-step = one panel of 64 input columns: the activation panel (256 rows x 128 bytes, whole cache
// lines) and the kept value blocks of its 16 units (unit u = member u / 2, block u % 2 of the panel;
// 2 KB each, staged at slot u) go to LDS by direct-to-LDS loads that every wave issues for its
// share. The 160 KB of LDS hold 3 activation stages and 2 value stages: during sub-step s the
// activation panel of s + 2 is loaded (issued during the first two 16-deep chunks of s) and the
// value blocks of s + 2 (during the last chunk, once the barrier has freed their stage). At the
// end of s every wave waits for its loads of s + 1 and a barrier publishes them.
// Groups whose every sub-step keeps all 16 units (e.g. block rows kept in full) run a body
// without presence tests; the others test each member's block before its products.
//   out tile^T [n][m] += A[n][k] . B[k][m],   B[k][m] = act[m][panel*64 + k]
//   forward:    A[n][k] = V[i][n][k]   (natural layout, 16-byte LDS reads)
//   input grad: A[n][k] = V[i][k][n]   (transposing LDS reads of the natural layout)
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <utility>
#include <vector>

#include "bsr_device.hpp"
#include "bsr_internal.hpp"

namespace bsr {
namespace {

using namespace dev;

constexpr int kXB = kWideRows * 128;                  // staged activation panel: 32 KB
constexpr int kWBB = 32 * 64;                          // one value block: 2 KB
constexpr int kVB = kWideU * kWBB;                     // staged value blocks of a panel: 32 KB
constexpr int kXStages = 3, kVStages = 2;
constexpr int kStagesBytes = kXStages * kXB + kVStages * kVB;   // 160 KB
constexpr int kOutPitch = kWideG * 32 * 2 + 16;        // staged output row (bytes)
constexpr int kSmem = kWideRows * kOutPitch > kStagesBytes ? kWideRows * kOutPitch : kStagesBytes;
static_assert(kSmem <= 160 * 1024, "LDS of one work-group");

struct WideArgs {
    const uint16_t *act;
    int in_ld, M;
    const uint16_t *V;
    uint32_t v_bytes;
    const uint16_t *bias;
    uint16_t *out;
    int out_ld;
};

// One work-group's tile: group g, activation tile mt0. DENSE: every sub-step keeps all 16 units.
template <bool TRANS, bool DENSE>
__device__ __forceinline__ void wide_tile(const WideArgs &a, const int32_t *__restrict__ sub_ptr,
                                           const int32_t *__restrict__ gout, const int32_t *__restrict__ rec, int g,
                                           int mt0, unsigned char *smem) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = wave & 1, wm = wave >> 1;   // rows 128 wr .., members 2 wm, 2 wm + 1
    const int l32 = lane & 31, lh = lane >> 5;

    const int rows = min(kWideRows, a.M - mt0 * kWideRows);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.act + (int64_t)mt0 * kWideRows * a.in_ld, (uint32_t)rows * a.in_ld * 2);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.V, a.v_bytes);
    const uint32_t sbase = lds_addr(smem);

    // Sub-step records come through scalar loads whose index is clamped into the group (no
    // select on the loaded values): a record is loaded three sub-steps ahead and first read at the
    // end of the sub-step that loaded it, when the wait for it costs nothing.
    struct Rec {
        int mask, blk[4];   // blk: value block of unit (wave + 8 j) / 2 (-1 = none)
        int segA, segB;     // byte offsets in an activation row of the panel's two input blocks
    };
    auto load_rec = [&](int s) __attribute__((always_inline)) {
        const int32_t *e = rec + (size_t)s * kWideRecInts;
        Rec x;
        x.mask = DENSE ? (1 << kWideU) - 1 : __builtin_amdgcn_readfirstlane(e[1]);
#pragma unroll
        for (int j = 0; j < 4; ++j) x.blk[j] = __builtin_amdgcn_readfirstlane(e[2 + ((wave + 8 * j) >> 1)]);
        x.segA = __builtin_amdgcn_readfirstlane(e[18]) * 64;
        x.segB = __builtin_amdgcn_readfirstlane(e[19]) * 64;
        return x;
    };
    // activation load i = wave + 8 j (j < 4) of the panel into activation stage xs: rows 8 i .. 8 i
    // + 7 (lane -> row 8 i + lane / 8, LDS chunk lane % 8 holding source chunk q = (lane % 8) ^
    // swz8(row): 16 bytes q % 4 of input block segA (q < 4) or segB). Rows past M read as zeros
    // through the range-checked voffset; a last half panel's missing block is never used.
    auto issue_x = [&](int xs, const Rec &x, int j) __attribute__((always_inline)) {
        const int i = wave + 8 * j;
        const int r = i * 8 + (lane >> 3);
        const int q = (lane & 7) ^ swz8(r);
        dma16(ra, sbase + (uint32_t)xs * kXB + (uint32_t)i * 1024u,
              (uint32_t)r * (uint32_t)a.in_ld * 2u + (uint32_t)(q < 4 ? x.segA : x.segB) + (uint32_t)((q & 3) << 4), 0);
    };
    // value load k = wave + 8 j (j < 4): half q = k % 2 of the block of unit u = k / 2 (if kept) into
    // value stage vs, 1 KB (lane -> block row 16 q + lane / 4, chunk (lane % 4) ^ swz4(row))
    auto issue_v = [&](int vs, const Rec &x, int j) __attribute__((always_inline)) {
        const int k = wave + 8 * j, u = k >> 1, q = k & 1;
        if (DENSE || ((x.mask >> u) & 1)) {
            const int n = 16 * q + (lane >> 2);
            dma16(rv, sbase + kXStages * kXB + (uint32_t)vs * kVB + (uint32_t)u * kWBB + (uint32_t)q * 1024u,
                  (uint32_t)(n * 64 + (((lane & 3) ^ swz4(n)) << 4)), (uint32_t)x.blk[j] * kWBB);
        }
    };

    f32x16 acc[4][2];   // [row tile][member of the wave]
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[rt][t][v] = 0.f;

    // value fragment of the block staged at wb for 16-deep chunk kc: natural layout for the
    // forward; for the input gradient lane l holds V[kc*16 + 8 (l / 32) .. + 7][l % 32], from two
    // transposing reads of 4 rows each
    auto wfrag = [&](const unsigned char *wb, int kc) __attribute__((always_inline)) {
        if constexpr (!TRANS) {
            return *reinterpret_cast<const bf16x8 *>(wb + l32 * 64 + (((2 * kc + lh) ^ swz4(l32)) << 4));
        } else {
            const int gq = lane >> 4, s16 = lane & 15;
            const int R = kc * 16 + (gq >> 1) * 8 + (s16 >> 2);
            const int C = (gq & 1) * 16 + 4 * (s16 & 3);
            auto at = [&](int row) {
                return (lds_i16x4 *)(wb + row * 64 + ((((C >> 3) ^ swz4(row)) << 4) | ((C & 7) << 1)));
            };
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(at(R));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(at(R + 4));
            const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            return __builtin_bit_cast(bf16x8, v);
        }
    };
    auto xfrag = [&](const unsigned char *xt, int rt, int c) __attribute__((always_inline)) {
        const int r = wr * 128 + rt * 32 + l32;
        return *reinterpret_cast<const bf16x8 *>(xt + r * 128 + (((2 * c + lh) ^ swz8(r)) << 4));
    };
    // Products of one staged sub-step, chunk by chunk (c = 16-deep chunk of the panel, block c / 2),
    // member by member: fragment set c & 1 holds chunk c. m4 = presence of this wave's 4 units (bit
    // 2 t + h: member 2 wm + t, block h of the panel). Absent units' products are skipped, never run
    // on zero blocks (zero times a non-finite activation is not zero). Fragments are read one chunk
    // ahead into the other register set (for every unit, present or not: a read of an unused slot
    // is harmless), so the LDS latency hides behind the matrix cores.
    bf16x8 xf[2][4], wf[2][2];
    auto read_frags = [&](int set, int xs, int vs, int c) __attribute__((always_inline)) {
        const unsigned char *xt = smem + xs * kXB;
        const unsigned char *wt = smem + kXStages * kXB + vs * kVB + wm * 4 * kWBB;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) xf[set][rt] = xfrag(xt, rt, c);
#pragma unroll
        for (int t = 0; t < 2; ++t) wf[set][t] = wfrag(wt + (2 * t + (c >> 1)) * kWBB, c & 1);
    };
    // the products of chunk c (presence bit 2 t + c / 2 of m4); after(t) runs after member t's
    auto products = [&](int c, int m4, auto &&after) __attribute__((always_inline)) {
        const int cur = c & 1, h = c >> 1;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            if (DENSE || ((m4 >> (2 * t + h)) & 1)) {
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) acc[rt][t] = mfma32(wf[cur][t], xf[cur][rt], acc[rt][t]);
            }
            __builtin_amdgcn_sched_barrier(0);
            after(t);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Sub-step pipeline. Before sub-step s: activation stages hold s, s + 1 (landed or in flight),
    // value stages s, s + 1; fragment set 0 holds chunk 0 of s. Sub-step s: chunks 0 .. 2 (each
    // reading the next chunk's fragments), with the activation panel of s + 2 issued between the
    // products of chunks 0 and 1 into the third activation stage (free since the last barrier);
    // then every wave waits for its LDS reads of s (all in registers now) and for its loads of
    // s + 1, and a barrier publishes s + 1 and frees the stages of s; then the value blocks of s + 2
    // are issued into their stage between the products of chunk 3, after the reads of chunk 0 of
    // s + 1. The barrier never waits on an LDS read, the next sub-step starts with its first
    // fragments in registers, and loads have about one sub-step to land.
    const int s0 = sub_ptr[g], s1 = sub_ptr[g + 1];
    if (s0 < s1) {
        Rec r0 = load_rec(s0), r1 = load_rec(min(s0 + 1, s1 - 1));
        Rec r2 = load_rec(min(s0 + 2, s1 - 1)), r3 = load_rec(min(s0 + 3, s1 - 1));
#pragma unroll
        for (int j = 0; j < 4; ++j) issue_x(0, r0, j);
#pragma unroll
        for (int j = 0; j < 4; ++j) issue_v(0, r0, j);
        if (s0 + 1 < s1) {
#pragma unroll
            for (int j = 0; j < 4; ++j) issue_x(1, r1, j);
#pragma unroll
            for (int j = 0; j < 4; ++j) issue_v(1, r1, j);
        }
        wait_vm<0, 0>(0);
        __syncthreads();
        read_frags(0, 0, 0, 0);
        int xs = 0, vs = 0;
        for (int s = s0; s < s1; ++s) {
            const int m4 = (r0.mask >> (4 * wm)) & 0xF;
            const bool more2 = s + 2 < s1;
            const int x2 = xs == 0 ? 2 : xs - 1;   // activation stage of s + 2 (that of s - 1)
#pragma unroll
            for (int c = 0; c < 3; ++c) {
                read_frags((c + 1) & 1, xs, vs, c + 1);
                // the 4 activation loads of s + 2 after the member groups of chunks 0 and 1
                products(c, m4, [&](int t) __attribute__((always_inline)) {
                    if (more2 && c < 2) issue_x(x2, r2, 2 * c + t);
                });
            }
            // every LDS read of sub-step s has landed in registers (chunk 3's included)
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            // the record of s + 4 is loaded now, with no LDS read outstanding: scalar loads share
            // the LDS wait counter and return out of order, so one in flight would turn the partial
            // LDS waits into full ones
            const Rec r4 = load_rec(min(s + 4, s1 - 1));
            // this wave's loads of s + 1 have landed; its 4 activation loads of s + 2 may not have
            if (more2) wait_vm<4, 4>(4);
            else wait_vm<0, 0>(0);
            __syncthreads();
            const int xn = xs == 2 ? 0 : xs + 1, vn = vs ^ 1;
            read_frags(0, xn, vn, 0);
            // the 4 value loads of s + 2, 2 per member group
            products(3, m4, [&](int t) __attribute__((always_inline)) {
                if (more2) {
                    issue_v(vs, r2, 2 * t);
                    issue_v(vs, r2, 2 * t + 1);
                }
            });
            r0 = r1;
            r1 = r2;
            r2 = r3;
            r3 = r4;
            xs = xn;
            vs = vn;
        }
    }
    __syncthreads();   // the stages are free for the output tile

    // Epilogue through LDS: item v of lane l of acc[rt][t] is output column 8 (v / 4) + 4 (l / 32) +
    // v % 4 of member 2 wm + t, activation row 128 wr + 32 rt + l % 32. Bias in fp32, one bf16
    // rounding; then every wave stores 32 staged rows as 16-byte pieces of whole 64-byte block rows.
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int tg = wm * 2 + t;
        const int o = gout[g * kWideG + tg];
        if (o < 0) continue;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int c = tg * 32 + q * 8 + lh * 4;
                const int row = wr * 128 + rt * 32 + l32;
                f32x4 v = quad(acc[rt][t], q);
                if (a.bias) v = add_bias4(v, a.bias + o * 32 + q * 8 + lh * 4);
                store4_bf16(reinterpret_cast<uint16_t *>(smem + row * kOutPitch + c * 2), v[0], v[1], v[2], v[3]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    __syncthreads();
    const int m0 = mt0 * kWideRows + wave * 32;
#pragma unroll 4
    for (int i = 0; i < 16; ++i) {
        const int seg = i * 64 + lane, row = seg >> 5, cs = seg & 31;   // 32 pieces per row
        const int t = cs >> 2, within = (cs & 3) * 8;
        const int o = gout[g * kWideG + t];
        if (o < 0 || m0 + row >= a.M) continue;
        const u32x4 val = *reinterpret_cast<const u32x4 *>(smem + (wave * 32 + row) * kOutPitch + cs * 16);
        __builtin_nontemporal_store(val, reinterpret_cast<u32x4 *>(a.out + (int64_t)(m0 + row) * a.out_ld + o * 32 + within));
    }
}

template <bool TRANS>
__global__ __launch_bounds__(512, 1) void k_wide_gemm(WideArgs a, const int32_t *__restrict__ order,
                                                  const int32_t *__restrict__ flags,
                                                  const int32_t *__restrict__ sub_ptr,
                                                  const int32_t *__restrict__ gout,
                                                  const int32_t *__restrict__ rec, int ngroups, int nmtiles, int tpc) {
    __shared__ __attribute__((aligned(1024))) unsigned char smem[kSmem];
    // Work-group -> (group, activation tile), as in the panel GEMM: each XCD takes a contiguous run
    // of chunks of tpc activation tiles x all groups (heaviest groups first), so the work-groups
    // running together on an XCD share activation panels and value blocks through its L2.
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int chunk = L / (tpc * ngroups), r4 = L % (tpc * ngroups);
    const int mc = min(tpc, nmtiles - tpc * chunk);
    const int g = order[r4 / mc];
    const int mt0 = tpc * chunk + r4 % mc;
    if (flags[g]) wide_tile<TRANS, true>(a, sub_ptr, gout, rec, g, mt0, smem);
    else wide_tile<TRANS, false>(a, sub_ptr, gout, rec, g, mt0, smem);
}

// ------------------------------------------------------------------------------------------
// 2:4 wide-tile forward (b = 32): the wide GEMM's tile, schedule, waves and pipeline with every kept
// block in the compressed 2:4 form (torchao sparsity README, Table 4.1: half the values plus 2-bit
// indices): Vc holds a block's 32 rows x 16 kept values (1 KB), meta its 32 rows x two 16-bit
// index words (128 bytes). Both are staged as they are: 1 KB of values per unit (identity lane map)
// and, per wave, the index words of its 2 units (u = wave + 8 t) by one load into its own 1 KB (lanes
// 8 t .. 8 t + 7 fetch unit u's 128 bytes, the others read zeros), so a sub-step stages 24 KB of
// values and indices instead of 32. Per block and row tile one v_smfmac_f32_32x32x32_bf16: lane
// (row n = l % 32, half h = l / 32) takes 8 kept values of columns 16 h .. 16 h + 15 of block row n
// and their 16 index bits; the activation operand is the two 16-deep fragments of the block's 32
// columns, read as one 16-element vector. Sub-step s: the block-0 products with the 4 activation
// loads of s + 2 among them, the wait and the barrier, then the block-1 products with the value and
// index loads of s + 2.
// ------------------------------------------------------------------------------------------
constexpr int kVB24 = kWideU * 1024 + 8 * 1024;                   // staged values + index words
constexpr uint32_t kPastEnd24 = 0xFFFFFFF0u;   // past both compressed arrays: such a load reads zeros
constexpr int kStages24 = kXStages * kXB + kVStages * kVB24;      // 144 KB
constexpr int kSmem24 = kWideRows * kOutPitch > kStages24 ? kWideRows * kOutPitch : kStages24;
static_assert(kSmem24 <= 160 * 1024, "LDS of one work-group");

struct WideArgs24 {
    const uint16_t *act;
    int in_ld, M;
    const uint16_t *Vc;
    uint32_t vc_bytes;
    const uint16_t *meta;
    uint32_t meta_bytes;
    const uint16_t *bias;
    uint16_t *out;
    int out_ld;
};

template <bool DENSE>
__device__ __forceinline__ void wide_tile_24(const WideArgs24 &a, const int32_t *__restrict__ sub_ptr,
                                             const int32_t *__restrict__ gout, const int32_t *__restrict__ rec, int g,
                                             int mt0, unsigned char *smem) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = wave & 1, wm = wave >> 1;   // rows 128 wr .., members 2 wm, 2 wm + 1
    const int l32 = lane & 31, lh = lane >> 5;

    const int rows = min(kWideRows, a.M - mt0 * kWideRows);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.act + (int64_t)mt0 * kWideRows * a.in_ld, (uint32_t)rows * a.in_ld * 2);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.Vc, a.vc_bytes);
    const __amdgpu_buffer_rsrc_t rm = make_rsrc(a.meta, a.meta_bytes);
    const uint32_t sbase = lds_addr(smem);
    const uint32_t vbase = sbase + kXStages * kXB;

    struct Rec {
        int mask, blk[2];   // blk: value block of unit wave + 8 t (-1 = none)
        int segA, segB;
    };
    auto load_rec = [&](int s) __attribute__((always_inline)) {
        const int32_t *e = rec + (size_t)s * kWideRecInts;
        Rec x;
        x.mask = DENSE ? (1 << kWideU) - 1 : __builtin_amdgcn_readfirstlane(e[1]);
#pragma unroll
        for (int t = 0; t < 2; ++t) x.blk[t] = __builtin_amdgcn_readfirstlane(e[2 + wave + 8 * t]);
        x.segA = __builtin_amdgcn_readfirstlane(e[18]) * 64;
        x.segB = __builtin_amdgcn_readfirstlane(e[19]) * 64;
        return x;
    };
    // activation load i = wave + 8 j (j < 4): as the wide GEMM
    auto issue_x = [&](int xs, const Rec &x, int j) __attribute__((always_inline)) {
        const int i = wave + 8 * j;
        const int r = i * 8 + (lane >> 3);
        const int q = (lane & 7) ^ swz8(r);
        dma16(ra, sbase + (uint32_t)xs * kXB + (uint32_t)i * 1024u,
              (uint32_t)r * (uint32_t)a.in_ld * 2u + (uint32_t)(q < 4 ? x.segA : x.segB) + (uint32_t)((q & 3) << 4), 0);
    };
    // kept values of unit u = wave + 8 t (if kept): 1 KB to unit slot u
    auto issue_v = [&](int vs, const Rec &x, int t) __attribute__((always_inline)) {
        const int u = wave + 8 * t;
        if (DENSE || ((x.mask >> u) & 1))
            dma16(rv, vbase + (uint32_t)vs * kVB24 + (uint32_t)u * 1024u, (uint32_t)lane * 16u, (uint32_t)x.blk[t] * 1024u);
    };
    // index words of this wave's units wave + 8 t: lanes 8 t .. 8 t + 7 load unit t's 128 bytes to
    // this wave's 1 KB (t * 128 ..); the other lanes and absent units read zeros
    auto issue_m = [&](int vs, const Rec &x) __attribute__((always_inline)) {
        const int t = (lane >> 3) & 1;
        const int blk = t == 0 ? x.blk[0] : x.blk[1];
        const uint32_t voff = lane < 16 && blk >= 0 ? (uint32_t)blk * 128u + (uint32_t)(lane & 7) * 16u : kPastEnd24;
        dma16(rm, vbase + (uint32_t)vs * kVB24 + kWideU * 1024u + (uint32_t)wave * 1024u, voff, 0);
    };

    f32x16 acc[4][2];   // [row tile][member of the wave]
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[rt][t][v] = 0.f;

    auto xfrag = [&](const unsigned char *xt, int rt, int c) __attribute__((always_inline)) {
        const int r = wr * 128 + rt * 32 + l32;
        return *reinterpret_cast<const bf16x8 *>(xt + r * 128 + (((2 * c + lh) ^ swz8(r)) << 4));
    };
    // fragments of block h of the panel: the activation fragments of its chunks 2 h, 2 h + 1, and the
    // kept values and index bits of each member t's unit u = 2 (2 wm + t) + h (present or not: a read
    // of an unused slot is harmless); unit u's index words sit in the region of wave u % 8, at
    // 128 (u / 8)
    bf16x16 xf[2][4];
    bf16x8 af[2][2];
    int ai[2][2];
    auto read_frags = [&](int set, int xs, int vs, int h) __attribute__((always_inline)) {
        const unsigned char *xt = smem + xs * kXB;
        const unsigned char *vt = smem + kXStages * kXB + vs * kVB24;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            xf[set][rt].lo = xfrag(xt, rt, 2 * h);
            xf[set][rt].hi = xfrag(xt, rt, 2 * h + 1);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int u = 2 * (2 * wm + t) + h;
            af[set][t] = *reinterpret_cast<const bf16x8 *>(vt + u * 1024 + l32 * 32 + lh * 16);
            ai[set][t] = *reinterpret_cast<const uint16_t *>(vt + kWideU * 1024 + (u & 7) * 1024 + (u >> 3) * 128 + l32 * 4 +
                                                             lh * 2);
        }
    };
    auto products = [&](int set, int h, int m4, auto &&after) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            if (DENSE || ((m4 >> (2 * t + h)) & 1)) {
#pragma unroll
                for (int rt = 0; rt < 4; ++rt)
                    acc[rt][t] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(af[set][t], xf[set][rt], acc[rt][t],
                                                                           ai[set][t], 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            after(t);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    const int s0 = sub_ptr[g], s1 = sub_ptr[g + 1];
    if (s0 < s1) {
        Rec r0 = load_rec(s0), r1 = load_rec(min(s0 + 1, s1 - 1));
        Rec r2 = load_rec(min(s0 + 2, s1 - 1)), r3 = load_rec(min(s0 + 3, s1 - 1));
#pragma unroll
        for (int j = 0; j < 4; ++j) issue_x(0, r0, j);
#pragma unroll
        for (int t = 0; t < 2; ++t) issue_v(0, r0, t);
        issue_m(0, r0);
        if (s0 + 1 < s1) {
#pragma unroll
            for (int j = 0; j < 4; ++j) issue_x(1, r1, j);
#pragma unroll
            for (int t = 0; t < 2; ++t) issue_v(1, r1, t);
            issue_m(1, r1);
        }
        wait_vm<0, 0>(0);
        __syncthreads();
        read_frags(0, 0, 0, 0);
        int xs = 0, vs = 0;
        for (int s = s0; s < s1; ++s) {
            const int m4 = (r0.mask >> (4 * wm)) & 0xF;
            const bool more2 = s + 2 < s1;
            const int x2 = xs == 0 ? 2 : xs - 1;   // activation stage of s + 2 (that of s - 1)
            read_frags(1, xs, vs, 1);
            // block 0's products with the 4 activation loads of s + 2 (2 per member group)
            products(0, 0, m4, [&](int t) __attribute__((always_inline)) {
                if (more2) {
                    issue_x(x2, r2, 2 * t);
                    issue_x(x2, r2, 2 * t + 1);
                }
            });
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            const Rec r4 = load_rec(min(s + 4, s1 - 1));
            // this wave's loads of s + 1 have landed; the 4 activation loads of s + 2 may be in flight
            if (more2) wait_vm<4, 4>(4);
            else wait_vm<0, 0>(0);
            __syncthreads();
            const int xn = xs == 2 ? 0 : xs + 1, vn = vs ^ 1;
            read_frags(0, xn, vn, 0);   // block 0 of s + 1 (harmless past the last sub-step)
            // block 1's products with the value and index loads of s + 2 (into the stage of s, free
            // since the barrier)
            products(1, 1, m4, [&](int t) __attribute__((always_inline)) {
                if (more2) {
                    issue_v(vs, r2, t);
                    if (t == 1) issue_m(vs, r2);
                }
            });
            r0 = r1;
            r1 = r2;
            r2 = r3;
            r3 = r4;
            xs = xn;
            vs = vn;
        }
    }
    __syncthreads();   // the stages are free for the output tile

#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int tg = wm * 2 + t;
        const int o = gout[g * kWideG + tg];
        if (o < 0) continue;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int c = tg * 32 + q * 8 + lh * 4;
                const int row = wr * 128 + rt * 32 + l32;
                f32x4 v = quad(acc[rt][t], q);
                if (a.bias) v = add_bias4(v, a.bias + o * 32 + q * 8 + lh * 4);
                store4_bf16(reinterpret_cast<uint16_t *>(smem + row * kOutPitch + c * 2), v[0], v[1], v[2], v[3]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    __syncthreads();
    const int m0 = mt0 * kWideRows + wave * 32;
#pragma unroll 4
    for (int i = 0; i < 16; ++i) {
        const int seg = i * 64 + lane, row = seg >> 5, cs = seg & 31;
        const int t = cs >> 2, within = (cs & 3) * 8;
        const int o = gout[g * kWideG + t];
        if (o < 0 || m0 + row >= a.M) continue;
        const u32x4 val = *reinterpret_cast<const u32x4 *>(smem + (wave * 32 + row) * kOutPitch + cs * 16);
        __builtin_nontemporal_store(val, reinterpret_cast<u32x4 *>(a.out + (int64_t)(m0 + row) * a.out_ld + o * 32 + within));
    }
}

__global__ __launch_bounds__(512, 1) void k_wide_gemm_24(WideArgs24 a, const int32_t *__restrict__ order,
                                                         const int32_t *__restrict__ flags,
                                                         const int32_t *__restrict__ sub_ptr,
                                                         const int32_t *__restrict__ gout,
                                                         const int32_t *__restrict__ rec, int ngroups, int nmtiles,
                                                         int tpc) {
    __shared__ __attribute__((aligned(1024))) unsigned char smem[kSmem24];
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int chunk = L / (tpc * ngroups), r4 = L % (tpc * ngroups);
    const int mc = min(tpc, nmtiles - tpc * chunk);
    const int g = order[r4 / mc];
    const int mt0 = tpc * chunk + r4 % mc;
    if (flags[g]) wide_tile_24<true>(a, sub_ptr, gout, rec, g, mt0, smem);
    else wide_tile_24<false>(a, sub_ptr, gout, rec, g, mt0, smem);
}

// ------------------------------------------------------------------------------------------
// Wide weight gradient (b = 32): for the kept blocks of a tile of 4 block rows x 16 block columns
// (any rows, any columns),
//   dV[i][p][q] = sum_m dY[m][r*32 + p] * X[m][c*32 + q]     (the block-masked SDDMM)
// over one chunk of activation rows. 8 waves, two per SIMD; wave w owns tile columns 2 w, 2 w + 1
// of all 4 rows: 4 x 2 accumulators of 32 x 32 (products D[q][p] += X^T . dY with A = X fragments
// and B = dY fragments, so each lane ends with 4 consecutive q of one p). Every one of the 64
// products is computed, absent blocks included, and only kept blocks are written: one code path,
// no per-block branches around the matrix-core chain. Per 32-row step, the 4 rows' dY segments
// (32 rows x 4 x 64 bytes, 8 KB) and the 16 columns' X segments (32 rows x 16 x 64 bytes, 16 KB
// ... 32 KB) are staged by direct-to-LDS loads, 4 stages deep (the 160 KB of LDS): the loads of
// step s + 4 are issued during step s, after every wave has read step s. A lane's source offset
// within a row is the same for every step, so it is computed once; the row part is a wave-uniform
// add. Loads past the chunk's rows read zeros (the buffer resources cover exactly the chunk's
// rows), which is also how the last steps' surplus loads stay harmless. Unused rows and columns
// of a tile read row or column 0: they only feed products that are dropped. Fragments come from
// transposing LDS reads; the 16-byte chunks of each staged row are XOR swizzled by 4 (row % 4),
// which keeps the reads of 4 consecutive rows per 16 lanes on distinct banks. Per 16-deep chunk a
// wave reads 2 + 4 fragments for 8 products.
// With one chunk of rows the sums are rounded to bf16 directly (staged through LDS, stored as
// 16-byte pieces of whole block rows); otherwise fp32 partials go to the workspace at the blocks'
// compact indices.
// ------------------------------------------------------------------------------------------
constexpr int kDwStep = 32;                        // activation rows per staged step
constexpr int kDwDYB = kDwStep * kWdwRows * 64;    // staged dY: 8 KB
constexpr int kDwXB = kDwStep * kWdwCols * 64;     // staged X: 32 KB
constexpr int kDwStage = kDwDYB + kDwXB;           // 40 KB
constexpr int kDwStages = 4;
static_assert(kDwStages * kDwStage <= 160 * 1024, "LDS of one work-group");
constexpr int kDwWaves8 = 8;                        // waves of a work-group, two per SIMD
constexpr int kDwLoads = (kDwDYB + kDwXB) / 1024 / kDwWaves8;   // direct-to-LDS loads per wave and step (5)
constexpr int kDwDYLoads = kDwDYB / 1024 / kDwWaves8;           // of which dY loads (1)

struct WdwOut {
    uint16_t *dV;       // bf16 blocks (one chunk of rows)
    float *partial;     // or fp32 partials [chunk][P2][1024] at compact index - cbase
    int ch, P2, cbase;
};

__device__ __forceinline__ void wide_dw_tile(const uint16_t *__restrict__ dY, int N, const uint16_t *__restrict__ X,
                                             int K, const int32_t *__restrict__ it, int m_begin, int rows,
                                             const WdwOut &o, unsigned char *smem) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, lh = lane >> 5;
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(dY + (size_t)m_begin * N, (uint32_t)((size_t)rows * N * 2));
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(X + (size_t)m_begin * K, (uint32_t)((size_t)rows * K * 2));
    const uint32_t sbase = lds_addr(smem);
    const int nsteps = (rows + kDwStep - 1) / kDwStep;

    // Loads of step `step` into stage st, 5 per wave (8 waves). dY load d = wave (1 KB: 4 activation
    // rows x 4 block rows x 64 bytes): lane -> activation row 4 d + lane / 16, staged chunk lane % 16
    // of that row, which holds source chunk (lane % 16) ^ 4 (lane / 16) (block row of the tile =
    // source chunk / 4, 16-byte piece = source chunk % 4). X loads x = wave + 8 k, k < 4 (one
    // activation row of 1 KB each): staged chunk lane holds source chunk lane ^ 4 (x % 4), x % 4 =
    // wave % 4 (tile column = source chunk / 4).
    const int dsrc = (lane & 15) ^ ((lane >> 4) << 2);
    const uint32_t dlane = (uint32_t)(lane >> 4) * (uint32_t)N * 2u + (uint32_t)max(it[dsrc >> 2], 0) * 64u +
                           (uint32_t)(dsrc & 3) * 16u;
    const int xsrc = lane ^ ((wave & 3) << 2);
    const uint32_t xlane = (uint32_t)max(it[4 + (xsrc >> 2)], 0) * 64u + (uint32_t)(xsrc & 3) * 16u;
    auto issue = [&](int st, int step, int k) __attribute__((always_inline)) {
        const uint32_t base = sbase + (uint32_t)st * kDwStage;
        if (k < kDwDYLoads) {
            const int d = wave + kDwWaves8 * k;
            dma16(rd, base + (uint32_t)d * 1024u, dlane + (uint32_t)(step * kDwStep + 4 * d) * (uint32_t)N * 2u, 0);
        } else {
            const int x = wave + kDwWaves8 * (k - kDwDYLoads);
            dma16(rx, base + kDwDYB + (uint32_t)x * 1024u, xlane + (uint32_t)(step * kDwStep + x) * (uint32_t)K * 2u, 0);
        }
    };

    // T[k0 + 8 (l / 32) .. + 7][n0 + l % 32] of a staged tile (rows of `pitch` bytes) for lane l:
    // two transposing reads of 4 rows (lane s of a 16-lane group points at row R + s / 4, columns
    // C .. C + 3: 8 bytes inside one 16-byte chunk)
    auto frag = [&](const unsigned char *tile, int pitch, int k0, int n0) __attribute__((always_inline)) {
        const int gq = lane >> 4, s16 = lane & 15;
        const int R = k0 + (gq >> 1) * 8 + (s16 >> 2);
        const int C = n0 + (gq & 1) * 16 + 4 * (s16 & 3);
        auto at = [&](int row) {
            return (lds_i16x4 *)(tile + row * pitch + ((((C >> 3) ^ ((row & 3) << 2)) << 4) | ((C & 7) << 1)));
        };
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(at(R));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(at(R + 4));
        const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return __builtin_bit_cast(bf16x8, v);
    };

    // wave w holds the blocks of all 4 rows x columns 2 w, 2 w + 1 of the tile (128 registers), two
    // waves per SIMD, so that one issues products while the other waits
    f32x16 acc[kWdwRows][2];   // [block row t][column jj of the wave]
#pragma unroll
    for (int t = 0; t < kWdwRows; ++t)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[t][jj][v] = 0.f;

    bf16x8 fa[2][2], fb[2][4];   // [set][jj]: X fragments (A); [set][t]: dY fragments (B)
    auto read_frags = [&](int set, int st, int kc) __attribute__((always_inline)) {
        const unsigned char *dt = smem + st * kDwStage, *xt = dt + kDwDYB;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) fa[set][jj] = frag(xt, kWdwCols * 64, kc * 16, (2 * wave + jj) * 32);
#pragma unroll
        for (int t = 0; t < kWdwRows; ++t) fb[set][t] = frag(dt, kWdwRows * 64, kc * 16, t * 32);
    };
    auto products = [&](int set, auto &&after) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < kWdwRows; ++t) {
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) acc[t][jj] = mfma32(fa[set][jj], fb[set][t], acc[t][jj]);
            __builtin_amdgcn_sched_barrier(0);
            after(t);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Step pipeline: before step s the stages hold steps s .. s + 3 (landed or in flight) and
    // fragment set 0 holds chunk 0 of s. Step s: read chunk 1, products of chunk 0 with the second
    // half of the loads of s + 3 issued in between (into the stage of s - 1, free since the last
    // barrier); wait for every LDS read of s and for this wave's loads of s + 1 (loads complete in
    // issue order, so those of s + 2 and s + 3 may stay in flight); barrier (s + 1 published, stage
    // of s free); read chunk 0 of s + 1; products of chunk 1 with the first half of the loads of
    // s + 4 issued in between into the stage of s. The issue of a direct-to-LDS load holds the wave
    // while the compute unit's load path is busy (about 64 bytes a clock), so the loads go out one or
    // two at a time between groups of 4 products. Steps past the chunk load zeros, so the loop has
    // no tail cases.
    // a step's 5 loads go out in two parts, 3 (the first 3 product groups of one half step) and 2
    constexpr int kHalf = 3;
    static_assert(kDwLoads == 5, "the product groups below issue 3 + 2 loads per step");
    auto spread = [&](int stage, int step, int k0, int nk) __attribute__((always_inline)) {
        return [=, &issue](int t) __attribute__((always_inline)) {
            if (t < nk) issue(stage, step, k0 + t);
        };
    };
#pragma unroll
    for (int q = 0; q < kDwStages; ++q)
#pragma unroll
        for (int k = 0; k < (q < kDwStages - 1 ? kDwLoads : kHalf); ++k) issue(q, q, k);
    // step 0 landed: the loads of steps 1 .. kDwStages - 2 and the first half of kDwStages - 1 may
    // stay in flight
    constexpr int kPrologueFlight = (kDwStages - 2) * kDwLoads + kHalf;
    wait_vm<kPrologueFlight, kPrologueFlight>(0);
    __syncthreads();
    read_frags(0, 0, 0);
    for (int s = 0; s < nsteps; ++s) {
        const int st = s % kDwStages;
        read_frags(1, st, 1);
        products(0, spread((s + kDwStages - 1) % kDwStages, s + kDwStages - 1, kHalf, kDwLoads - kHalf));
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        wait_vm<(kDwStages - 2) * kDwLoads, (kDwStages - 2) * kDwLoads>(0);
        __syncthreads();
        read_frags(0, (s + 1) % kDwStages, 0);
        products(1, spread(st, s + kDwStages, 0, kHalf));
    }
    wait_vm<0, 0>(0);
    __syncthreads();   // the stages are free for the output staging

    // Item v of lane l of acc[t][jj]: D[q][p] with q = 8 (v / 4) + 4 (l / 32) + v % 4 (block column
    // of dV), p = l % 32 (block row): 4 consecutive q of one p.
    if (o.partial) {
#pragma unroll
        for (int t = 0; t < kWdwRows; ++t)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int c = it[kWdwCompactAt + 16 * t + 2 * wave + jj];
                if (c < 0) continue;
                float *dst = o.partial + ((size_t)o.ch * o.P2 + (c - o.cbase)) * 1024 + l32 * 32 + 4 * lh;
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) *reinterpret_cast<f32x4 *>(dst + 8 * q4) = quad(acc[t][jj], q4);
                __builtin_amdgcn_sched_barrier(0);
            }
        return;
    }
    // bf16: wave's 8 blocks staged as [slot 2 t + jj][32 rows][64 + 16 bytes], then 16-byte stores
    constexpr int BP = 80;                          // staged block row pitch (bytes)
    static_assert(kDwWaves8 * 8 * 32 * BP <= kDwStages * kDwStage, "output staging fits in the stages");
    unsigned char *wst = smem + wave * 8 * 32 * BP;
#pragma unroll
    for (int t = 0; t < kWdwRows; ++t)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 v = quad(acc[t][jj], q4);
                store4_bf16(reinterpret_cast<uint16_t *>(wst + (2 * t + jj) * 32 * BP + l32 * BP + (8 * q4 + 4 * lh) * 2),
                            v[0], v[1], v[2], v[3]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    // (each wave reads back only what it wrote: no barrier needed beyond the wave's own LDS ordering)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll 4
    for (int i = 0; i < 16; ++i) {
        const int seg = i * 64 + lane, slot = seg >> 7, rowp = (seg >> 2) & 31, piece = seg & 3;
        const int e = it[kWdwBlockAt + 16 * (slot >> 1) + 2 * wave + (slot & 1)];
        if (e < 0) continue;
        const u32x4 val = *reinterpret_cast<const u32x4 *>(wst + slot * 32 * BP + rowp * BP + piece * 16);
        *reinterpret_cast<u32x4 *>(o.dV + (size_t)e * 1024 + rowp * 32 + piece * 8) = val;
    }
}

// Thin weight-gradient item: up to 8 blocks anywhere, wave w computes block w over one chunk of
// activation rows, dV[i][p][q] = sum_m dY[m][r*32 + p] * X[m][c*32 + q] (the block-masked SDDMM),
// with no reuse between the blocks and no exchange between the waves (no barrier). Per 32-row step a
// wave stages its block's dY segment and X segment (32 rows x 64 bytes each, 4 direct-to-LDS loads
// of 16 rows: lane -> row lane / 4, 16-byte piece lane % 4) in its own 4 KB of a stage; 5 stages, so
// that the loads of a step are issued 4 steps ahead (these blocks' segments mostly miss L2, and one
// block's products do not cover a miss). Rows past the chunk read zeros, as in the tile items; the
// wave drains its loads before it ends, so that none lands in the LDS of a later work-group.
constexpr int kThinStages = 5;
constexpr int kThinWaveBytes = 2 * kDwStep * 64;                 // dY and X segments of one step: 4 KB
constexpr int kThinStage = kDwWaves8 * kThinWaveBytes;          // 32 KB
static_assert(kWdwThinBlocks == kDwWaves8, "one wave per block of a thin item");
static_assert(kThinStages * kThinStage <= kDwStages * kDwStage, "thin stages fit the tile items' LDS");

__device__ __forceinline__ void wide_dw_thin(const uint16_t *__restrict__ dY, int N, const uint16_t *__restrict__ X,
                                             int K, const int32_t *__restrict__ it, int m_begin, int rows,
                                             const WdwOut &o, unsigned char *smem) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, lh = lane >> 5;
    const int e = it[kWdwBlockAt + wave];
    if (e < 0) return;   // wave-uniform; the thin path has no barrier
    const int r = it[12 + wave], c = it[4 + wave];
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(dY + (size_t)m_begin * N, (uint32_t)((size_t)rows * N * 2));
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(X + (size_t)m_begin * K, (uint32_t)((size_t)rows * K * 2));
    const uint32_t sbase = lds_addr(smem) + (uint32_t)wave * kThinWaveBytes;
    unsigned char *const mine = smem + wave * kThinWaveBytes;
    const int nsteps = (rows + kDwStep - 1) / kDwStep;
    const uint32_t dlane = (uint32_t)(lane >> 2) * (uint32_t)N * 2u + (uint32_t)r * 64u + (uint32_t)(lane & 3) * 16u;
    const uint32_t xlane = (uint32_t)(lane >> 2) * (uint32_t)K * 2u + (uint32_t)c * 64u + (uint32_t)(lane & 3) * 16u;
    auto issue = [&](int st, int step) __attribute__((always_inline)) {
        const uint32_t base = sbase + (uint32_t)st * kThinStage;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t row = (uint32_t)(step * kDwStep + 16 * h);
            dma16(rd, base + (uint32_t)h * 1024u, dlane + row * (uint32_t)N * 2u, 0);
            dma16(rx, base + 2048u + (uint32_t)h * 1024u, xlane + row * (uint32_t)K * 2u, 0);
        }
    };
    // T[k0 + 8 (l / 32) .. + 7][l % 32] of a staged 32 x 64-byte segment for lane l: two transposing
    // reads of 4 rows (lane s of a 16-lane group points at row R + s / 4, columns C .. C + 3)
    auto frag = [&](const unsigned char *seg, int k0) __attribute__((always_inline)) {
        const int gq = lane >> 4, s16 = lane & 15;
        const int R = k0 + (gq >> 1) * 8 + (s16 >> 2);
        const int C = (gq & 1) * 16 + 4 * (s16 & 3);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(seg + R * 64 + C * 2));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(seg + (R + 4) * 64 + C * 2));
        const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return __builtin_bit_cast(bf16x8, v);
    };
    f32x16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
    for (int q = 0; q < kThinStages - 1; ++q) issue(q, q);
    for (int s = 0; s < nsteps; ++s) {
        // into the stage of s - 1, once every LDS read of s - 1 has returned
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        issue((s + kThinStages - 1) % kThinStages, s + kThinStages - 1);
        wait_vm<4 * (kThinStages - 1), 4 * (kThinStages - 1)>(0);   // this wave's loads of s have landed
        const unsigned char *seg = mine + (s % kThinStages) * kThinStage;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) acc = mfma32(frag(seg + 2048, kc * 16), frag(seg, kc * 16), acc);
    }
    wait_vm<0, 0>(0);
    // item v of lane l: D[q][p], q = 8 (v / 4) + 4 (l / 32) + v % 4 (block column), p = l % 32
    if (o.partial) {
        float *dst = o.partial + ((size_t)o.ch * o.P2 + (it[kWdwCompactAt + wave] - o.cbase)) * 1024 + l32 * 32 + 4 * lh;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) *reinterpret_cast<f32x4 *>(dst + 8 * q4) = quad(acc, q4);
    } else {
        uint16_t *dst = o.dV + (size_t)e * 1024 + l32 * 32 + 4 * lh;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 v = quad(acc, q4);
            store4_bf16(dst + 8 * q4, v[0], v[1], v[2], v[3]);
        }
    }
}

// Work-groups go to the XCDs round robin (XCD = blockIdx % 8), so that each XCD gets an equal
// share of both kinds of work in its first round: XCD x runs, in order, its contiguous run of the
// first n1 items (whole rows range each), then its contiguous run of the n2 x c2 (chunk, item) pairs
// of the other items (items fastest). Work-groups past an XCD's share exit at once.
__global__ __launch_bounds__(512, 1) void k_wide_dw(const uint16_t *__restrict__ dY, int N, const uint16_t *__restrict__ X,
                                                    int K, int M, const int32_t *__restrict__ items, int n1, int n2,
                                                    int c2, int mchunk, int cbase, int P2,
                                                    float *__restrict__ partial, uint16_t *__restrict__ dV) {
    __shared__ __attribute__((aligned(1024))) unsigned char smem[kDwStages * kDwStage];
    const int x = blockIdx.x % kXCDs, i = blockIdx.x / kXCDs;
    const int a0 = (int)((int64_t)n1 * x / kXCDs), a = (int)((int64_t)n1 * (x + 1) / kXCDs) - a0;
    int item, m_begin = 0, rows = M;
    WdwOut o{dV, nullptr, 0, P2, cbase};
    if (i < a) {
        item = a0 + i;
    } else {
        const int64_t n2c = (int64_t)n2 * c2;
        const int64_t b0 = n2c * x / kXCDs, b = n2c * (x + 1) / kXCDs - b0;
        const int64_t j = i - a;
        if (j >= b) return;
        const int64_t g = b0 + j;
        o.ch = (int)(g / n2);
        item = n1 + (int)(g % n2);
        m_begin = o.ch * mchunk;
        rows = min(M - m_begin, mchunk);
        if (c2 > 1) o.partial = partial;
    }
    const int32_t *it = items + (size_t)item * kWdwItemInts;
    if (it[kWdwKindAt] == 1) wide_dw_thin(dY, N, X, K, it, m_begin, rows, o, smem);
    else wide_dw_tile(dY, N, X, K, it, m_begin, rows, o, smem);
}

// dV of the blocks of the split items: the fixed-order sum of their fp32 partials over the chunks.
// Thread = 4 values of one block (compact index cbase + c).
__global__ __launch_bounds__(256) void k_wide_dw_reduce(const float *__restrict__ partial, int nchunks, int P2,
                                                        int cbase, const int32_t *__restrict__ compact,
                                                        uint16_t *__restrict__ dV) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)P2 * 256) return;
    const int64_t c = idx >> 8, v = (idx & 255) * 4;
    const size_t stride = (size_t)P2 * 1024;
    const float *src = partial + c * 1024 + v;
    f32x4 s = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(src));
    for (int ch = 1; ch < nchunks; ++ch)
        s += __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(src + (size_t)ch * stride));
    store4_bf16(dV + (size_t)compact[cbase + c] * 1024 + v, s[0], s[1], s[2], s[3]);
}

// Activation tiles per XCD chunk: 4 for the forward, 2 for the input gradient, whose 16 groups on
// the Zipf layer (16384 x 4096 -> 11008) walk the same panels, so that a chunk's work-groups all run
// together on one XCD (warm, two runs: 4 tiles 489 / 493 us, 2 tiles 482 / 479; forward 479 / 474
// against 490 / 494).
int wide_tiles_per_chunk(int nmtiles, bool transposed) {
    int t = transposed ? 2 : 4;
    if (const char *f = std::getenv("BSR_WIDE_TPC")) t = std::atoi(f);   // tuning knob
    return std::max(1, std::min(t, nmtiles));
}

}  // namespace

bool use_wide(const bsr_pattern &p, bool transposed, int64_t M) {
    if (p.b != 32 || p.device_built) return false;
    const WideSchedule &s = transposed ? p.wide_bwd : p.wide_fwd;
    if (const char *f = std::getenv("BSR_GEMM_VARIANT")) return std::atoi(f) == kGemmVariants;   // tuning knob
    const int64_t nsub = s.nsub();
    if (nsub == 0 || M < kWideRows) return false;
    // dense groups: on average at least half of a sub-step's 16 units keep a block
    return (double)s.nunits >= 8.0 * (double)nsub;
}

// Splits of the wide weight-gradient items for M activation rows. A model of one XCD (32 compute
// units, one work-group each, work-groups placed in order on the unit that frees first) gives the
// finishing time, in 32-row steps of a dense item, of its share of the first n1 items (whole:
// ceil(M / 32) steps each) and of the (chunk, item) pairs of the rest (mchunk / 32 steps each, items
// fastest), plus a few steps per work-group for its prologue and epilogue. A step of a gathered item
// costs 1.3 dense steps, one of a thin item 0.8 (Zipf layer, 4 chunks: 769 ns per dense step, 1179
// per gathered, 628 per thin). Partials of split items: written during the products, read once by
// the reduction (counted as 1.5 times their bytes at ~4 MB per step), plus its launch. The
// candidates keep the dense items whole, or split every item, into 1 .. 16 chunks of at least 256
// rows; the cheapest wins (ties: fewer chunks). The plan is cached per pattern for the last M.
static WideDwPlan plan_wide_dw_model(const bsr_pattern &p, int64_t M) {
    const WideDwSchedule &s = p.wdw;
    WideDwPlan best;
    if (s.n == 0 || M <= 0) return best;
    constexpr int64_t kExtra = 6;   // prologue and epilogue of a work-group, in steps
    constexpr int kUnits = kCUs / kXCDs;
    const int64_t steps = (M + 31) / 32;
    // step cost of each item relative to a dense one
    std::vector<double> cost(s.n, 1.0);
    for (int k = s.ndense; k < s.n; ++k) cost[k] = s.items[(size_t)k * kWdwItemInts + kWdwKindAt] == 1 ? 0.8 : 1.3;
    std::vector<std::pair<double, int64_t>> free_at;   // (time, units), at most kUnits entries
    auto place = [&](int64_t jobs, double len) {      // on the units that free first, in order
        while (jobs > 0) {
            size_t k = 0;
            for (size_t q = 1; q < free_at.size(); ++q)
                if (free_at[q].first < free_at[k].first) k = q;
            const double t = free_at[k].first;
            const int64_t use = std::min(jobs, free_at[k].second);
            if (use == free_at[k].second) free_at.erase(free_at.begin() + (long)k);
            else free_at[k].second -= use;
            bool merged = false;
            for (auto &f : free_at)
                if (f.first == t + len) f.second += use, merged = true;
            if (!merged) free_at.push_back({t + len, use});
            jobs -= use;
        }
    };
    // the XCD's a whole items, then its (chunk, item) pairs b0 .. b0 + b - 1 (item n1 + pair % n2), in
    // runs of equal cost
    auto xcd_time = [&](int64_t a, int n1, int64_t b0, int64_t b, int n2, int64_t csteps) {
        free_at.assign(1, {0.0, (int64_t)kUnits});
        place(a, (double)(steps + kExtra));
        for (int64_t g = b0; g < b0 + b;) {
            const double c = cost[n1 + (int)(g % n2)];
            int64_t e = g + 1;
            while (e < b0 + b && cost[n1 + (int)(e % n2)] == c) ++e;
            place(e - g, (double)csteps * c + (double)kExtra);
            g = e;
        }
        double last = 0;
        for (auto &f : free_at) last = std::max(last, f.first);
        return last;
    };
    double best_cost = 0;
    bool have = false;
    for (int n1 : {s.ndense, 0}) {
        if (have && n1 == 0 && s.ndense == 0) break;
        for (int c2 = 1; c2 <= 16; ++c2) {
            const int64_t mchunk = ((M + c2 - 1) / c2 + 31) / 32 * 32;
            if (c2 > 1 && mchunk < 256) break;
            const int c2e = (int)((M + mchunk - 1) / mchunk);
            if (c2 > 1 && c2e != c2) continue;
            const int n2 = s.n - n1;
            double t = 0;
            for (int x = 0; x < kXCDs; ++x) {
                const int64_t a0 = (int64_t)n1 * x / kXCDs, a = (int64_t)n1 * (x + 1) / kXCDs - a0;
                const int64_t n2c = (int64_t)n2 * c2e;
                const int64_t b0 = n2c * x / kXCDs, b = n2c * (x + 1) / kXCDs - b0;
                t = std::max(t, xcd_time(a, n1, b0, b, n2 > 0 ? n2 : 1, mchunk / 32));
            }
            const int64_t P2 = s.first[s.n] - s.first[n1];
            const double cost = (double)t + (c2e > 1 ? (double)P2 * c2e * 6144.0 / 4.0e6 + 8.0 : 0.0);
            if (!have || cost < best_cost) {
                have = true;
                best_cost = cost;
                best.n1 = n1;
                best.n2 = n2;
                best.c2 = c2e;
                best.mchunk = (int)(c2e > 1 ? mchunk : M);
                best.cbase = s.first[n1];
                best.P2 = (int)P2;
            }
            if (n2 == 0) break;
        }
    }
    return best;
}

WideDwPlan plan_wide_dw(const bsr_pattern &p, int64_t M) {
    const WideDwSchedule &s = p.wdw;
    WideDwPlan best;
    bool cached = false;
    {
        std::lock_guard<std::mutex> lock(p.wdw_plan_mu);
        if (p.wdw_plan_M == M) best = p.wdw_plan, cached = true;
    }
    if (!cached) {
        best = plan_wide_dw_model(p, M);
        std::lock_guard<std::mutex> lock(p.wdw_plan_mu);
        p.wdw_plan_M = M;
        p.wdw_plan = best;
    }
    if (const char *f = std::getenv("BSR_WDW_SPLIT")) {   // tuning knob: "n1,c2"
        int n1 = 0, c2 = 1;
        if (std::sscanf(f, "%d,%d", &n1, &c2) == 2 && n1 >= 0 && n1 <= s.n && c2 >= 1) {
            const int64_t mchunk = ((M + c2 - 1) / c2 + 31) / 32 * 32;
            best.n1 = n1;
            best.n2 = s.n - n1;
            best.c2 = (int)((M + mchunk - 1) / mchunk);
            best.mchunk = (int)(best.c2 > 1 ? mchunk : M);
            best.cbase = s.first[n1];
            best.P2 = s.first[s.n] - s.first[n1];
        }
    }
    return best;
}

int32_t launch_wide_dw(const bsr_pattern &p, const DwArgs &a, const WideDwPlan &w, float *partial, void *stream) {
    if (p.wdw.n == 0) return BSR_OK;
    const hipStream_t st = (hipStream_t)stream;
    int most = 0;
    for (int x = 0; x < kXCDs; ++x) {
        const int64_t n2c = (int64_t)w.n2 * w.c2;
        const int64_t share = (int64_t)w.n1 * (x + 1) / kXCDs - (int64_t)w.n1 * x / kXCDs + n2c * (x + 1) / kXCDs -
                              n2c * x / kXCDs;
        most = (int)std::max<int64_t>(most, share);
    }
    if (most == 0) return BSR_OK;
    hipLaunchKernelGGL(k_wide_dw, dim3((unsigned)(most * kXCDs)), dim3(kDwWaves8 * 64), 0, st, a.dY, p.N, a.X, p.K, (int)a.M,
                       p.dev.wdw_items, w.n1, w.n2, w.c2, w.mchunk, w.cbase, w.P2, partial, a.dV);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(BSR_ERR_HIP, std::string("wide weight-gradient launch: ") + hipGetErrorString(e));
    if (w.c2 > 1 && w.P2 > 0) {
        hipLaunchKernelGGL(k_wide_dw_reduce, dim3((unsigned)(((int64_t)w.P2 * 256 + 255) / 256)), dim3(256), 0, st,
                           partial, w.c2, w.P2, w.cbase, p.dev.wdw_compact, a.dV);
        e = hipGetLastError();
        if (e != hipSuccess) return fail(BSR_ERR_HIP, std::string("wide weight-gradient reduce: ") + hipGetErrorString(e));
    }
    return BSR_OK;
}

int32_t launch_wide_gemm_24(const bsr_pattern &p, const FwdArgs &a, const uint16_t *Vc, const uint16_t *meta,
                            void *stream) {
    const hipStream_t st = (hipStream_t)stream;
    const WideSchedule &s = p.wide_fwd;
    const DevSchedule &d = p.dev.wide_fwd;
    const int nmtiles = (int)((a.M + kWideRows - 1) / kWideRows);
    const int64_t nwg = (int64_t)s.ngroups * nmtiles;
    if (nwg > (int64_t)INT32_MAX) return fail(BSR_ERR_INVALID_ARG, "problem too large for one launch");
    if ((size_t)p.nnzb * 1024 >= (size_t)kPastEnd24) return fail(BSR_ERR_INVALID_ARG, "compressed values above 4 GiB");
    if ((int64_t)kWideRows * a.in_ld * 2 + 256 > (int64_t)UINT32_MAX)
        return fail(BSR_ERR_INVALID_ARG, "activation rows too long for 32-bit buffer offsets");
    if (nwg == 0) return BSR_OK;
    const int tpc = wide_tiles_per_chunk(nmtiles, false);
    const WideArgs24 wa{a.act, a.in_ld, (int)a.M, Vc, (uint32_t)((size_t)p.nnzb * 1024), meta,
                        (uint32_t)((size_t)p.nnzb * 128), a.bias, a.out, a.out_ld};
    hipLaunchKernelGGL(k_wide_gemm_24, dim3((unsigned)nwg), dim3(512), 0, st, wa, d.order, d.flags, d.sub_ptr, d.out,
                       d.rec, s.ngroups, nmtiles, tpc);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(BSR_ERR_HIP, std::string("wide 2:4 gemm launch: ") + hipGetErrorString(e));
    return BSR_OK;
}

int32_t launch_wide_gemm(const bsr_pattern &p, bool transposed, const FwdArgs &a, void *stream) {
    const hipStream_t st = (hipStream_t)stream;
    const WideSchedule &s = transposed ? p.wide_bwd : p.wide_fwd;
    const DevSchedule &d = transposed ? p.dev.wide_bwd : p.dev.wide_fwd;
    const int nmtiles = (int)((a.M + kWideRows - 1) / kWideRows);
    const int64_t nwg = (int64_t)s.ngroups * nmtiles;
    if (nwg > (int64_t)INT32_MAX) return fail(BSR_ERR_INVALID_ARG, "problem too large for one launch");
    if ((size_t)p.nnzb * 32 * 32 * 2 > (size_t)UINT32_MAX) return fail(BSR_ERR_INVALID_ARG, "block values above 4 GiB");
    if ((int64_t)kWideRows * a.in_ld * 2 + 256 > (int64_t)UINT32_MAX)
        return fail(BSR_ERR_INVALID_ARG, "activation rows too long for 32-bit buffer offsets");
    if (nwg == 0) return BSR_OK;
    const int tpc = wide_tiles_per_chunk(nmtiles, transposed);
    const WideArgs wa{a.act, a.in_ld, (int)a.M, a.V, (uint32_t)((size_t)p.nnzb * 32 * 32 * 2), a.bias, a.out, a.out_ld};
    if (transposed)
        hipLaunchKernelGGL(k_wide_gemm<true>, dim3((unsigned)nwg), dim3(512), 0, st, wa, d.order, d.flags, d.sub_ptr,
                           d.out, d.rec, s.ngroups, nmtiles, tpc);
    else
        hipLaunchKernelGGL(k_wide_gemm<false>, dim3((unsigned)nwg), dim3(512), 0, st, wa, d.order, d.flags, d.sub_ptr,
                           d.out, d.rec, s.ngroups, nmtiles, tpc);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(BSR_ERR_HIP, std::string("wide gemm launch: ") + hipGetErrorString(e));
    return BSR_OK;
}

}  // namespace bsr
