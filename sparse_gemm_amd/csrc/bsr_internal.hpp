// bsr_internal.hpp -- library-internal types shared by the host code and the kernel launchers.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <mutex>
#include <vector>

#include "bsr_linear.h"

namespace bsr {

// Panel GEMM (forward and input gradient). The activations are consumed in panels of 64
// columns (128 bytes of bf16 per row, one full cache line), so a panel covers 64 / b input blocks
// (2 for b = 32, 1 for b = 64). A work-group owns G output blocks (block rows of W for the
// forward, block columns for the input gradient) and 32 activation rows per wave; its work list
// is the panels in which its members have kept blocks. A member's kept block inside a panel is a
// "unit" (unit u = member * (64 / b) + block within the panel). Each sub-step stages one panel of
// activations and at most S value blocks ("slots"); a panel with more kept blocks than S takes
// several sub-steps.
constexpr int kPanelCols = 64;
// Kernel variants (members per group G, slots per sub-step S, compute waves per work-group; each
// variant has its own work lists, since S decides how panels split into sub-steps):
//   0: G = 4, S = 8 (all 8 units of a panel), 8 waves (256 activation rows) -- large problems;
//   1: G = 4, S = 4, 4 waves (128 rows, three LDS stages: 2 work-groups per CU);
//   2: G = 2, S = 4 (all 4 units), 4 waves (two LDS stages: 3 work-groups per CU);
//   3: G = 1, S = 2 (both units), 4 waves (two LDS stages) -- when too few groups of 2 to fill.
// For b = 64 every variant has G = S = 1 (one 64 x 64 block per panel). Every work-group also has
// waves that only issue the loads: panel_loader_waves(compute waves) of them. Each load into LDS
// takes a wave tens of cycles to issue while the memory system is busy, so more issuing waves
// deliver more bytes per clock (measured: 2 -> 4 -> 8 loaders for 8 compute waves).
constexpr int kGemmVariants = 4;
constexpr int panel_loader_waves(int compute_waves) { return compute_waves == 8 ? 8 : 4; }
// Loader waves of the weight-gradient kernel.
constexpr int kLoaderWaves = 2;
struct GemmVariant {
    int G, S, waves;
};
// The variant whose work lists a device-built pattern's rebuild produces (G = 4, S = 4, 4 waves
// for b = 32; one block per panel, 4 waves for b = 64).
constexpr int kDeviceVariant = 1;
inline GemmVariant gemm_variant(int b, int k) {
    if (b == 64) return GemmVariant{1, 1, k == 0 ? 8 : 4};
    return k == 0 ? GemmVariant{4, 8, 8} : k == 1 ? GemmVariant{4, 4, 4} : k == 2 ? GemmVariant{2, 4, 4} : GemmVariant{1, 2, 4};
}

// Sub-step record, kRecInts ints: [0] panel index; [1 + k] value block in slot k (-1 = empty),
// k < S; [1 + S + w] slot of units 8w .. 8w + 7, 4 bits each (unit u at bits 4 * (u % 8); 15 =
// the unit has no block in this sub-step).
constexpr int kRecInts = 16;
struct GroupSchedule {
    int G = 0, S = 0;
    int ngroups = 0;
    int64_t npanels = 0;             // (group, panel) pairs with kept blocks; sub-steps / npanels > 1
                                     // when panels hold more units than S
    std::vector<int32_t> order;      // processing order of the groups (most sub-steps first)
    std::vector<int32_t> sub_ptr;    // [ngroups + 1]
    std::vector<int32_t> out;        // [ngroups * G] output block index per member, -1 = unused
    std::vector<int32_t> rec;        // [nsub * kRecInts]
};

// Wide-tile panel GEMM (b = 32; the matrix-core-bound regime of dense groups): a work-group owns
// kWideG = 8 output blocks (256 output columns) and 256 activation rows, held by 8 waves as 4 x 2
// grids of 32 x 32 accumulators. One sub-step per 64-column panel in which any member keeps a
// block; the value block of unit u (member u / 2, block u % 2 of the panel) is staged at slot u.
// Record, kWideRecInts ints: [0] panel, [1] presence mask (bit u = unit u has a block),
// [2 + u] value block of unit u (-1 = none), [18], [19] the panel's two input blocks (the
// activation columns 32 [18] .. + 31 and 32 [19] .. + 31 staged as its 64 columns; consecutive
// blocks for the forward, blocks paired by kept-block count for the input gradient).
constexpr int kWideG = 8;
constexpr int kWideU = 16;
constexpr int kWideRecInts = 20;
constexpr int kWideRows = 256;
struct WideSchedule {
    int ngroups = 0;
    int64_t nunits = 0;              // kept blocks over all sub-steps (= nnzb)
    std::vector<int32_t> order;      // processing order of the groups (most sub-steps first)
    std::vector<int32_t> sub_ptr;    // [ngroups + 1]
    std::vector<int32_t> out;        // [ngroups * kWideG] output block per member, -1 = unused
    std::vector<int32_t> rec;        // [nsub * kWideRecInts]
    std::vector<int32_t> flags;      // [ngroups]: 1 = dense group (every sub-step keeps all 16 units)
    int64_t nsub() const { return sub_ptr.empty() ? 0 : sub_ptr.back(); }
};

// Weight-gradient work items. A tile is TR consecutive block rows by TC consecutive block columns
// (TR * b = 256 and TC * b = 512 columns: per activation row, 512 bytes of dY and 1 KB of X, whole
// cache lines); an item is up to kDwWaves * dw_slots(b) of a tile's kept blocks, each compute wave
// owning up to dw_slots(b) of them. Item layout, kDwItemInts ints: [0] first block row, [1] first
// block column, [2 + w] number of blocks of compute wave w, [16 + 8 w + q] block q of wave w:
// (CSR index << 8) | (row in the tile << 4) | column in the tile.
constexpr int kDwWaves = 6;
constexpr int kDwItemInts = 80;
inline int dw_tile_rows(int b) { return 256 / b; }
inline int dw_tile_cols(int b) { return 512 / b; }
inline int dw_slots(int b) { return b == 64 ? 2 : 8; }
struct DwSchedule {
    int n = 0;
    std::vector<int32_t> items;   // [n * kDwItemInts], by super-tiles of 8 x 4 tiles
};

// Wide weight-gradient items (b = 32). Tile items: kWdwRows block rows (any rows) by kWdwCols block
// columns (any columns), run by 8 waves that each hold 4 x 2 block accumulators; the products of
// absent blocks are computed and dropped. Three kinds, in this order: dense items (4 rows whose 16
// consecutive columns are all kept, rows taken in order of decreasing kept-block count, so that
// full rows share tiles); gathered items (a seed row, most remaining blocks, with the 3 rows that
// share most of its columns, and the 16 columns most of the 4 rows keep) that keep at least
// kWdwThinBelow blocks; then thin items, the blocks of the sparser gathered tiles in order of
// (column, row), kWdwThinBlocks at a time, one wave each (see make_wide_dw). Tile item layout,
// kWdwItemInts ints: [t] block row t (t < 4; -1 = unused), [4 + j] block column j (j < 16; -1 =
// unused), [kWdwKindAt] -1, [kWdwBlockAt + 16 t + j] CSR index of block (t, j) or -1,
// [kWdwCompactAt + 16 t + j] its compact index (blocks numbered in item order, row-major inside an
// item) or -1. Thin item: [kWdwKindAt] 1, block k (k < kWdwThinBlocks) in column [4 + k] and row
// [12 + k], CSR index [kWdwBlockAt + k] (-1 = none), compact index [kWdwCompactAt + k]; every other
// entry -1.
constexpr int kWdwRows = 4;
constexpr int kWdwCols = 16;
constexpr int kWdwKindAt = 20;
constexpr int kWdwBlockAt = 24;
constexpr int kWdwCompactAt = 88;
constexpr int kWdwItemInts = 152;
constexpr int kWdwWindow = 32;      // candidate rows per gathered item (next by remaining count)
constexpr int kWdwThinBlocks = 8;   // blocks of a thin item
constexpr int kWdwThinBelow = 16;   // gathered tiles keeping fewer blocks become thin items
struct WideDwSchedule {
    int n = 0;        // items
    int ndense = 0;   // the first ndense items are dense
    std::vector<int32_t> items;     // [n * kWdwItemInts], dense items in XCD-friendly order
    std::vector<int32_t> compact;   // [nnzb]: CSR index of compact index c
    std::vector<int32_t> first;     // [n + 1]: compact index of each item's first block; nnzb
};

// How one weight-gradient call runs the wide items: the first n1 whole (one work-group each over
// every activation row), the other n2 split into c2 chunks of mchunk rows whose fp32 partials (P2
// blocks per chunk, compact indices cbase ..) a reduction sums.
struct WideDwPlan {
    int n1 = 0, n2 = 0, c2 = 1, mchunk = 0, cbase = 0, P2 = 0;
};

struct DevSchedule {
    const int32_t *order = nullptr, *sub_ptr = nullptr, *out = nullptr, *rec = nullptr;
    const int32_t *flags = nullptr;   // wide schedules: per group, 1 = every sub-step keeps all units
};

// Device copies of the metadata (one allocation, carved into arrays).
struct DeviceMeta {
    void *base = nullptr;
    size_t bytes = 0;
    int device = -1;
    const int32_t *row_ptr = nullptr, *col_idx = nullptr, *col_ptr = nullptr, *row_idx = nullptr,
                  *perm = nullptr;
    DevSchedule fwd[kGemmVariants], bwd[kGemmVariants];
    DevSchedule wide_fwd, wide_bwd;
    const int32_t *dw_items = nullptr;
    const int32_t *wdw_items = nullptr, *wdw_compact = nullptr;
    // device-built patterns: the live block count and weight-gradient item count, the builders'
    // scratch and the metadata rebuild's workspace
    const int32_t *live_nnzb = nullptr, *live_items = nullptr;
    void *sched_scratch = nullptr, *rebuild_ws = nullptr;
    const int32_t *small_m_rows = nullptr;  // small-M forward: [R][4] {block row, first block, end
                                            // block, 0}, most blocks first
    const int32_t *small_m_work = nullptr;  // balanced small-M work list: [n][4] {block row, first
                                            // block, end block, first slice | slices << 8}
};

}  // namespace bsr

struct bsr_pattern {
    int32_t N = 0, K = 0, b = 0, R = 0, C = 0, nnzb = 0;
    std::vector<int32_t> row_ptr, col_idx, col_ptr, row_idx, perm, small_m_rows, small_m_work;
    bsr::GroupSchedule fwd[bsr::kGemmVariants], bwd[bsr::kGemmVariants];
    bsr::WideSchedule wide_fwd, wide_bwd;   // b = 32 only (empty otherwise)
    bsr::DwSchedule dw;        // items of the blocks the wide items leave
    bsr::WideDwSchedule wdw;   // b = 32 only
    bsr::DeviceMeta dev;
    bool uploaded = false;
    // Device-built pattern (bsr_pattern_create_device): metadata and work lists live on the device
    // only, rebuilt there from a device mask; nnzb is the capacity (the most kept blocks it holds),
    // dw.n the capacity of weight-gradient items, and no host-side list is filled.
    bool device_built = false;
    // The wide weight-gradient split of the last M planned (the plan depends on the pattern and M
    // only; a call plans it twice, for the workspace size and for the launch).
    mutable std::mutex wdw_plan_mu;
    mutable int64_t wdw_plan_M = -1;
    mutable bsr::WideDwPlan wdw_plan;
};

namespace bsr {

// Most kept blocks a pattern may hold: the weight-gradient work items pack a block's CSR
// position into the upper 23 bits of an int32 (position << 8 | tile coordinates).
constexpr int32_t kMaxNnzb = (1 << 23) - 1;

// Builds CSR-derived metadata and schedules from validated CSR arrays (nnzb <= kMaxNnzb).
void build_pattern(bsr_pattern &p);

// Canonical CSR of a row-major R x C block mask (nonzero = kept).
void csr_from_mask(int32_t R, int32_t C, const uint8_t *mask, std::vector<int32_t> &row_ptr,
                   std::vector<int32_t> &col_idx);

// Checks host CSR arrays of an R x C block grid: nullptr when they are canonical (row_ptr starts
// at 0, is non-decreasing and ends at nnzb; columns in range and strictly increasing in a row),
// else a static description of the first defect.
const char *check_csr(int32_t R, int32_t C, int32_t nnzb, const int32_t *row_ptr, const int32_t *col_idx);

// Records an error message for the calling thread and returns `status` (bsr_error.cpp).
int32_t fail(int32_t status, const std::string &msg);
// The calling thread's last message ("" if none).
const char *last_error();

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
// Whether the wide-tile kernel takes this call (dense groups, enough rows).
bool use_wide(const bsr_pattern &p, bool transposed, int64_t M);
int32_t launch_wide_gemm(const bsr_pattern &p, bool transposed, const FwdArgs &a, void *stream);
// the wide forward with 2:4-compressed blocks (Vc [nnzb][32][16], meta [nnzb][32][2])
int32_t launch_wide_gemm_24(const bsr_pattern &p, const FwdArgs &a, const uint16_t *Vc, const uint16_t *meta,
                            void *stream);
// sparse24: forward only; a.V holds 2:4 block images (bsr_values_pack_24) instead of bf16 blocks,
// or with meta24 the kept values of the compressed form (meta24: its index words).
int32_t launch_group_gemm(const bsr_pattern &p, bool transposed, const FwdArgs &a, void *stream,
                          bool sparse24 = false, const uint16_t *meta24 = nullptr);
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
// Comma-separated names of the main kernels one call of op (0 forward, 1 input gradient, 2 weight
// gradient, bias gradient excluded) launches for M rows; small_max: the forward's small-M limit.
std::string kernels_of(const bsr_pattern &p, int op, int64_t M, int64_t small_max);
int32_t launch_dw(const bsr_pattern &p, const DwArgs &a, void *stream);
// The wide weight-gradient items (bsr_wide.hip): fp32 partials [chunk][nnzb][b*b] when partial
// is not null, else bf16 into a.dV.
WideDwPlan plan_wide_dw(const bsr_pattern &p, int64_t M);
int32_t launch_wide_dw(const bsr_pattern &p, const DwArgs &a, const WideDwPlan &w, float *partial, void *stream);
// Device address of the current device's BSR_NOALLOC_SCRATCH_BYTES scratch array (looked up
// once per device; no allocation).
int32_t noalloc_scratch(void **out);

// Compute units the balanced small-M work list is laid out for (one MI355X).
constexpr int kSmallMUnits = 256;

// Rows at or below this count take the small-M (streaming) forward kernel.
constexpr int64_t kSmallM = 16;

}  // namespace bsr
