// bsr_internal.hpp -- library-internal types shared by the host code and the kernel launchers.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "bsr_linear.h"

namespace bsr {

// Output blocks per work-group of the forward / input-gradient kernels. Each pattern keeps two
// work lists: a wide one (more output blocks share every activation tile that is loaded) and a
// narrow one (more work-groups, for shapes that would not fill the chip otherwise).
inline int wide_group(int b) { return b == 64 ? 4 : 8; }
inline int narrow_group(int b) { return b == 64 ? 2 : 4; }
// Kept blocks of one block row handled by one weight-gradient work-group.
inline int dw_group(int b) { return b == 64 ? 2 : 4; }

// Host-built work list of the forward or input-gradient kernel. Output blocks (block rows of W
// for the forward, block columns for the input gradient) are grouped G at a time; a group's
// steps are the union of the input blocks its members touch, padded with empty steps to a
// multiple of P (the prefetch depth of the kernel, which processes P steps per loop trip).
// Per step s the kernel reads one record of RS ints, laid out for what it issues at step s:
//   rec[s*RS + 0]      bit t set = member t has a kept block at step s
//   rec[s*RS + 1]      input block of step s + P (activations prefetched at step s)
//   rec[s*RS + 2 + t]  value block of member t at step s + P (prefetched at step s), -1 = none
// and per group one header of HS ints: the input blocks of its first P steps, then the value
// blocks of those steps (P runs of G, -1 = none). Past the last real step, input blocks repeat
// the last real one and value blocks are -1.
struct GroupSchedule {
    int G = 0, P = 0, RS = 0, HS = 0;
    int ngroups = 0;
    std::vector<int32_t> order;      // processing order of the groups (most steps first)
    std::vector<int32_t> step_ptr;   // [ngroups + 1], padded steps
    std::vector<int32_t> out;        // [ngroups * G] output block index per slot, -1 = unused
    std::vector<int32_t> rec;        // [nsteps * RS]
    std::vector<int32_t> hdr;        // [ngroups * HS]
};

// Prefetch depth (steps per loop trip) of the group GEMM for block size b (compile-time tuning
// knobs BSR_GEMM_DEPTH32 / BSR_GEMM_DEPTH64).
#ifndef BSR_GEMM_DEPTH32
#define BSR_GEMM_DEPTH32 3
#endif
#ifndef BSR_GEMM_DEPTH64
#define BSR_GEMM_DEPTH64 2
#endif
constexpr int gemm_depth(int b) { return b == 64 ? BSR_GEMM_DEPTH64 : BSR_GEMM_DEPTH32; }
constexpr int pow2_at_least(int n) { return n <= 4 ? 4 : n <= 8 ? 8 : n <= 16 ? 16 : n <= 32 ? 32 : 64; }
// Ints per step record and per group header, for G members and depth P (at most 64: one wave
// lane per int).
constexpr int rec_stride(int G) { return pow2_at_least(G + 2); }
constexpr int hdr_stride(int G, int P) { return pow2_at_least(P + P * G); }

// Host-built work list of the weight-gradient kernel: runs of up to GB consecutive kept blocks
// of one block row (they share the block row's slab of dY), most blocks first.
struct DwSchedule {
    int GB = 0;
    int ngroups = 0;
    std::vector<int32_t> row, first, count;   // [ngroups] each
};

struct DevSchedule {
    const int32_t *order = nullptr, *step_ptr = nullptr, *out = nullptr, *rec = nullptr, *hdr = nullptr;
};

// Device copies of the metadata (one allocation, carved into arrays).
struct DeviceMeta {
    void *base = nullptr;
    size_t bytes = 0;
    int device = -1;
    const int32_t *row_ptr = nullptr, *col_idx = nullptr, *col_ptr = nullptr, *row_idx = nullptr,
                  *perm = nullptr;
    DevSchedule fwd[2], bwd[2];   // [0] wide groups, [1] narrow groups
    const int32_t *dw_row = nullptr, *dw_first = nullptr, *dw_count = nullptr;
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
