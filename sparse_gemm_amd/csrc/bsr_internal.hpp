// bsr_internal.hpp -- library-internal types shared by the host code and the kernel launchers.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "bsr_linear.h"

namespace bsr {

// Group GEMM shapes. A work-group (8 waves x 32 activation rows) computes G output
// blocks (block rows of W for the forward, block columns for the input gradient). A group's steps
// are the input blocks its members touch; each step is cut into sub-steps of at most S kept blocks
// (S == G: "direct" sub-steps, slot t = member t). Candidate (G, S) pairs per block size; the
// pattern builder keeps, for each of the two G, the S with the fewest estimated load instructions.
// Work-groups of 8 waves (256 activation rows) by default; the narrow groups also come in a
// 4-wave (128-row) form, for problems too small to fill the chip with the larger tiles.
constexpr int kGemmWaves = 8;
constexpr int gemm_wave_rows(int) { return 32; }
constexpr int gemm_rows(int b) { return kGemmWaves * gemm_wave_rows(b); }
constexpr int kGemmWavesSmall = 4;
inline int wide_group(int b) { return b == 64 ? 2 : 8; }
inline int narrow_group(int b) { return b == 64 ? 1 : 4; }
// Slots per sub-step the kernels are instantiated for, per (b, G).
inline std::vector<int> gemm_slot_options(int b, int G) {
    if (b == 32) return G == 8 ? std::vector<int>{2, 4, 8} : std::vector<int>{2, 4};
    return G == 2 ? std::vector<int>{1, 2} : std::vector<int>{1};
}

// Host-built work list of the forward or input-gradient kernel. Sub-steps are padded per group to
// a multiple of P (the kernel's prefetch depth: it handles P sub-steps per loop trip). Record of
// sub-step s, RS ints: rec[s*RS] = input block; rec[s*RS + 1 + k] = slot k: for S < G,
// (value block << 5) | member, for S == G the value block of member k; -1 = empty. Padding
// sub-steps repeat the group's last input block and have empty slots.
struct GroupSchedule {
    int G = 0, S = 0, P = 0, RS = 0;
    int ngroups = 0;
    std::vector<int32_t> order;      // processing order of the groups (most sub-steps first)
    std::vector<int32_t> sub_ptr;    // [ngroups + 1]
    std::vector<int32_t> out;        // [ngroups * G] output block index per member, -1 = unused
    std::vector<int32_t> rec;        // [nsub * RS]
};

// Prefetch depth (sub-steps per loop trip) of the group GEMM for block size b, G members and S
// slots (compile-time tuning knobs; the shapes with the most registers in use get the shallower).
#ifndef BSR_GEMM_DEPTH32
#define BSR_GEMM_DEPTH32 3
#endif
#ifndef BSR_GEMM_DEPTH64
#define BSR_GEMM_DEPTH64 2
#endif
constexpr int gemm_depth(int b, int G, int S) {
    return (b == 64 || (G == 8 && S == 8)) ? BSR_GEMM_DEPTH64 : BSR_GEMM_DEPTH32;
}
constexpr int pow2_at_least(int n) { return n <= 4 ? 4 : n <= 8 ? 8 : n <= 16 ? 16 : n <= 32 ? 32 : 64; }
constexpr int rec_stride(int S) { return pow2_at_least(1 + S); }

// Weight-gradient work items. An item is a set of up to TR block rows and up to TC block
// columns; it computes every kept block where they cross, and stages each row's dY slab and each
// column's X slab once per chunk of M, so a slab is shared by all the item's blocks in its row or
// column. "Dense" items (TR x TC = 8 x 8 for b = 32, 4 x 4 for b = 64) take row groups' columns
// that hold kept blocks in at least half of the group's rows; "runs" (one row, up to 4 (b = 32)
// or 2 (b = 64) columns) take the remaining blocks. Item layout, TS ints: rows[TR] (-1 unused),
// cols[TC] (-1 unused), blk[TR*TC] (CSR index of the kept block at (row i, column j), -1 if none).
struct DwShape {
    int TR, TC;
    constexpr int TS() const { return (TR + TC + TR * TC + 15) / 16 * 16; }
};
constexpr DwShape dw_dense_shape(int b) { return b == 64 ? DwShape{4, 4} : DwShape{8, 8}; }
constexpr DwShape dw_runs_shape(int b) { return b == 64 ? DwShape{1, 2} : DwShape{1, 4}; }

struct DwItems {
    int n = 0;
    std::vector<int32_t> items;   // [n * TS]
};
struct DwSchedule {
    DwItems dense, runs;
    std::vector<int32_t> cmap;                       // [nnzb] index of the block within its kind
    std::vector<int32_t> dense_blocks, run_blocks;   // CSR index of each kind's blocks, by that index
};

struct DevSchedule {
    const int32_t *order = nullptr, *sub_ptr = nullptr, *out = nullptr, *rec = nullptr;
};

// Device copies of the metadata (one allocation, carved into arrays).
struct DeviceMeta {
    void *base = nullptr;
    size_t bytes = 0;
    int device = -1;
    const int32_t *row_ptr = nullptr, *col_idx = nullptr, *col_ptr = nullptr, *row_idx = nullptr,
                  *perm = nullptr;
    DevSchedule fwd[2], bwd[2];   // [0] wide groups, [1] narrow groups
    const int32_t *dw_dense = nullptr, *dw_runs = nullptr, *dw_cmap = nullptr, *dw_dense_blocks = nullptr,
                  *dw_run_blocks = nullptr;
    const int32_t *rows_by_nnz = nullptr;   // small-M forward: block rows, most blocks first
};

}  // namespace bsr

struct bsr_pattern {
    int32_t N = 0, K = 0, b = 0, R = 0, C = 0, nnzb = 0;
    std::vector<int32_t> row_ptr, col_idx, col_ptr, row_idx, perm, rows_by_nnz;
    bsr::GroupSchedule fwd[2], bwd[2];   // [0] wide groups, [1] narrow groups
    bsr::DwSchedule dw;
    bsr::DeviceMeta dev;
    bool uploaded = false;
};

namespace bsr {

// Builds CSR-derived metadata and schedules from validated CSR arrays.
void build_pattern(bsr_pattern &p);

// Records an error message for the calling thread and returns `status`.
int32_t fail(int32_t status, const std::string &msg);

// ---- kernel launchers (bsr_kernels.hip). All return a bsr_status. ----
struct FwdArgs {
    const uint16_t *act;   // [M][in_ld]
    int64_t M;
    int in_ld;
    const uint16_t *V;
    const uint16_t *bias;  // may be null
    uint16_t *out;         // [M][out_ld]
    int out_ld;
};
int32_t launch_group_gemm(const bsr_pattern &p, bool transposed, const FwdArgs &a, void *stream);
int32_t launch_small_m_fwd(const bsr_pattern &p, const FwdArgs &a, void *stream);

struct DwArgs {
    const uint16_t *dY;
    const uint16_t *X;
    int64_t M;
    uint16_t *dV;
    uint16_t *dbias;
    void *ws;
    size_t ws_bytes;
};
size_t dw_workspace_bytes(const bsr_pattern &p, int64_t M);
int32_t launch_dw(const bsr_pattern &p, const DwArgs &a, void *stream);

// Rows at or below this count take the small-M (streaming) forward kernel.
constexpr int64_t kSmallM = 16;

}  // namespace bsr
