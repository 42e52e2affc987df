// bsr_internal.hpp -- library-internal types shared by the host code and the kernel launchers.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "bsr_linear.h"

namespace bsr {

// Group size (output blocks handled by one work-group) of the forward / input-gradient
// kernels, per block size. One step of a group reads one input block column (forward) or
// block row (input gradient) of the activations and multiplies it into every output block
// of the group that has a kept block there.
constexpr int kGroupFor32 = 4;
constexpr int kGroupFor64 = 2;
inline int group_size(int b) { return b == 64 ? kGroupFor64 : kGroupFor32; }

// A host-built work list for the forward or input-gradient kernel.
struct GroupSchedule {
    int G = 0;                       // output blocks per group
    int ngroups = 0;
    std::vector<int32_t> order;      // processing order of the groups (most steps first)
    std::vector<int32_t> step_ptr;   // [ngroups + 1]
    std::vector<int32_t> out;        // [ngroups * G] output block index per slot, -1 = unused
    std::vector<int32_t> step_in;    // [nsteps] input block index of each step
    std::vector<int32_t> step_blk;   // [nsteps * G] value-block index per slot, -1 = absent
};

// Device copies of the metadata (one allocation, carved into arrays).
struct DeviceMeta {
    void *base = nullptr;
    size_t bytes = 0;
    int device = -1;
    const int32_t *row_ptr = nullptr, *col_idx = nullptr, *col_ptr = nullptr, *row_idx = nullptr,
                  *perm = nullptr, *blk_row = nullptr;
    // forward schedule
    const int32_t *f_order = nullptr, *f_step_ptr = nullptr, *f_out = nullptr, *f_step_in = nullptr,
                  *f_step_blk = nullptr;
    // input-gradient schedule
    const int32_t *t_order = nullptr, *t_step_ptr = nullptr, *t_out = nullptr, *t_step_in = nullptr,
                  *t_step_blk = nullptr;
    // small-M forward: block rows, most blocks first
    const int32_t *rows_by_nnz = nullptr;
};

}  // namespace bsr

struct bsr_pattern {
    int32_t N = 0, K = 0, b = 0, R = 0, C = 0, nnzb = 0;
    std::vector<int32_t> row_ptr, col_idx, col_ptr, row_idx, perm, blk_row, rows_by_nnz;
    bsr::GroupSchedule fwd, bwd;  // forward (groups of block rows), input grad (groups of block columns)
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
