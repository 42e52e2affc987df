/*
 * bsr_linear.h -- C ABI of the block-sparse linear layer on AMD Instinct MI355X (gfx950).
 *
 * The layer is a drop-in replacement for a dense linear layer (pytorch_block_sparse
 * summary page, "Block-Sparse Implementation and Usage": BlockSparseLinear replaces
 * torch.nn.Linear and takes a density at construction). Its weight W[N,K] (out x in)
 * keeps a pattern of dense b x b blocks that is fixed at initialisation (same page,
 * "Future Development Roadmap"). The weight is stored as BSR (pytorch/ao sparsity
 * README, Table 4.1): dense blocks plus the block coordinates, here as a CSR index
 * pointer over block rows (row_ptr), the block column of every kept block (col_idx),
 * and the block values V. The backward pass also walks the transposed (CSC) form of
 * the same pattern: col_ptr, row_idx and perm.
 *
 * Notation: R = N/b block rows, C = K/b block columns, nnzb = kept blocks.
 *   row_ptr[R+1]  int32  first CSR position of each block row; row_ptr[R] = nnzb
 *   col_idx[nnzb] int32  block column of each kept block, ascending inside a row
 *   col_ptr[C+1]  int32  first CSC position of each block column; col_ptr[C] = nnzb
 *   row_idx[nnzb] int32  block row of each kept block in CSC order, ascending in a column
 *   perm[nnzb]    int32  CSR position of the j-th block in CSC order
 *   V[nnzb][b][b] bf16   V[i][p][q] = W[r*b + p][col_idx[i]*b + q] for i in row r
 *
 * What the calls compute: the results equal dense matmul with the zero-filled weight
 * W~ (pytorch/ao sparsity README, workflow section: sparse and dense matmul with zeros
 * in the missing places are numerically equivalent):
 *   bsr_linear_fwd         Y  = X . W~^T + bias
 *   bsr_linear_bwd_input   dX = dY . W~
 *   bsr_linear_bwd_weight  dV[i] = block (r, col_idx[i]) of dY^T . X, for kept blocks
 *                          only (the README's out-of-place mask update dW' = dW (Mask)),
 *                          and optionally dbias = column sums of dY.
 *
 * Conventions for every call:
 *   - bf16 is passed as its raw 16-bit pattern (bsr_bf16). Arithmetic: bf16 inputs,
 *     fp32 accumulation, one round-to-nearest-even to bf16 per output element.
 *   - Activations and gradients are dense, row-major, contiguous device buffers owned by
 *     the caller: X[M][K], Y[M][N], dY[M][N], dX[M][K]. Device pointers must be 16-byte
 *     aligned (BSR_ERR_MISALIGNED otherwise).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Compute calls
 *     only enqueue work on it and return; nothing is synchronised.
 *   - Arguments are checked before anything is enqueued; on any error nothing is
 *     written and the call returns a nonzero bsr_status; bsr_last_error() then holds a
 *     message for the calling thread.
 *   - A pattern is immutable after creation, so calls with one pattern may run on
 *     several streams at once. The pattern's device metadata lives on the device that
 *     was current at creation; compute calls must run with that device current.
 *   - No C++ exception crosses this interface.
 *   - Size limits (BSR_ERR_INVALID_ARG beyond them): at most 2^23 - 1 kept blocks per
 *     pattern (checked at creation); 32-bit buffer offsets in the kernels: V below 4 GiB,
 *     256 rows of X (forward) or dY (input gradient) below 4 GiB, and for the weight
 *     gradient (M + 32) rows of dY and of X each below 4 GiB.
 */
#ifndef BSR_LINEAR_H
#define BSR_LINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BSR_ABI_VERSION 1

typedef uint16_t bsr_bf16;              /* raw bfloat16 bits */
typedef struct bsr_pattern bsr_pattern; /* opaque, owned by the library */

enum bsr_status {
    BSR_OK = 0,
    BSR_ERR_INVALID_ARG = 1,        /* null pointer, bad size, malformed CSR, ... */
    BSR_ERR_UNSUPPORTED = 2,        /* block size other than 32 or 64 */
    BSR_ERR_MISALIGNED = 3,         /* a device pointer not 16-byte aligned */
    BSR_ERR_WORKSPACE_TOO_SMALL = 4,
    BSR_ERR_HIP = 5,                /* a HIP runtime call or kernel launch failed */
    BSR_ERR_OUT_OF_MEMORY = 6,
    BSR_ERR_NO_DEVICE_DATA = 7      /* compute call on a host-only pattern */
};

/* Version of this interface (BSR_ABI_VERSION of the built library). */
int32_t bsr_abi_version(void);

/* Build a pattern from a block mask (pytorch/ao sparsity README, workflow section: the
 * hand-off format is a dense weight with zeros; its block mask says which b x b blocks
 * are kept).
 *   N, K   weight shape (out, in); both multiples of b, both > 0.
 *   b      block size: 32 or 64 (BSR_ERR_UNSUPPORTED otherwise).
 *   mask   host array [N/b][K/b], row-major; nonzero byte = kept block. Read only
 *          during the call.
 *   upload 1: copy the metadata to the current HIP device (synchronously; the only
 *          host-to-device copy the library makes). 0: host-only pattern, usable for
 *          bsr_pattern_info / bsr_pattern_export but not for compute calls.
 *   out    receives the new pattern; the caller releases it with bsr_pattern_destroy.
 * Blocks are ordered canonically: ascending column inside a row (CSR) and ascending row
 * inside a column (CSC). */
int32_t bsr_pattern_create_from_mask(int32_t N, int32_t K, int32_t b, const uint8_t *mask,
                                     int32_t upload, bsr_pattern **out);

/* Build a pattern from host CSR arrays: the index pointer and block indices of the BSR
 * format (pytorch/ao sparsity README, Table 4.1), e.g. to restore a saved pattern, which
 * stays fixed once chosen (pytorch_block_sparse summary page, "Future Development
 * Roadmap"). row_ptr[N/b+1] must start at 0, be non-decreasing and end at nnzb;
 * col_idx[nnzb] must lie in [0, K/b) and be strictly increasing inside each row
 * (BSR_ERR_INVALID_ARG otherwise). */
int32_t bsr_pattern_create_from_csr(int32_t N, int32_t K, int32_t b, int32_t nnzb,
                                    const int32_t *row_ptr, const int32_t *col_idx,
                                    int32_t upload, bsr_pattern **out);

/* Shape of a pattern (the weight's N x K, the block size b and the number of kept blocks
 * of the BSR format, pytorch/ao sparsity README, Table 4.1); any output pointer may be
 * NULL. Host only, no device access. */
int32_t bsr_pattern_info(const bsr_pattern *p, int32_t *N, int32_t *K, int32_t *b,
                         int32_t *nnzb);

/* Copy the metadata to caller-owned host arrays sized row_ptr[R+1], col_idx[nnzb],
 * col_ptr[C+1], row_idx[nnzb], perm[nnzb]: the CSR index pointer and indices and their
 * transposed (CSC) form (pytorch/ao sparsity README, Table 4.1), with perm mapping CSC
 * order to CSR positions. Any pointer may be NULL (skipped). Host only. */
int32_t bsr_pattern_export(const bsr_pattern *p, int32_t *row_ptr, int32_t *col_idx,
                           int32_t *col_ptr, int32_t *row_idx, int32_t *perm);

/* Release a pattern (the fixed block pattern of one layer, pytorch_block_sparse summary
 * page, "Future Development Roadmap") and its device metadata. The caller guarantees
 * that no enqueued work still uses it (for example by synchronising the streams it was
 * used on).
 * NULL is ignored. */
void bsr_pattern_destroy(bsr_pattern *p);

/* Forward: Y[M][N] = X[M][K] . W~^T + bias (pytorch_block_sparse summary page, usage:
 * the nn.Linear forward with the block-sparse weight).
 *   X     device [M][K] bf16.
 *   M     rows of X and Y, >= 0 (M = 0 returns BSR_OK and enqueues nothing).
 *   V     device [nnzb][b][b] bf16 block values in CSR order.
 *   bias  device [N] bf16, or NULL for no bias.
 *   Y     device [M][N] bf16 output; every element is written (rows of W~ with no kept
 *         block give bias, or 0). Must not overlap X, V or bias. */
int32_t bsr_linear_fwd(const bsr_pattern *p, const bsr_bf16 *X, int64_t M, const bsr_bf16 *V,
                       const bsr_bf16 *bias, bsr_bf16 *Y, void *stream);

/* Input gradient: dX[M][K] = dY[M][N] . W~ (same contract as the forward, with the
 * transposed pattern). The kernels walk the CSC metadata; no atomics, so the result is
 * deterministic. Columns of W~ with no kept block give 0.
 *   dY    device [M][N] bf16;  V as for the forward;  dX device [M][K] bf16 output. */
int32_t bsr_linear_bwd_input(const bsr_pattern *p, const bsr_bf16 *dY, int64_t M,
                             const bsr_bf16 *V, bsr_bf16 *dX, void *stream);

/* Bytes of device workspace bsr_linear_bwd_weight needs for M rows (may be 0). */
size_t bsr_linear_bwd_weight_workspace(const bsr_pattern *p, int64_t M);

/* Weight gradient on the kept blocks only (pytorch/ao sparsity README, criteria list:
 * out-of-place update dW' = dW (Mask)):
 *   dV[i][p][q] = sum over m < M of dY[m][r*b + p] * X[m][col_idx[i]*b + q].
 *   dY     device [M][N] bf16;  X device [M][K] bf16.
 *   dV     device [nnzb][b][b] bf16 output, same order and layout as V.
 *   dbias  device [N] bf16 output (column sums of dY), or NULL to skip.
 *   workspace / ws_bytes  caller-owned device scratch of at least
 *          bsr_linear_bwd_weight_workspace(p, M) bytes (BSR_ERR_WORKSPACE_TOO_SMALL
 *          otherwise); may be NULL when that size is 0. Its contents on entry do not
 *          matter; it must not be used by other work until this call's work is done.
 * With M = 0 the gradients are zero: dV and dbias are filled with 0. Summation runs in
 * fp32 over all of M in a fixed order, so the result is deterministic. */
int32_t bsr_linear_bwd_weight(const bsr_pattern *p, const bsr_bf16 *dY, const bsr_bf16 *X,
                              int64_t M, bsr_bf16 *dV, bsr_bf16 *dbias, void *workspace,
                              size_t ws_bytes, void *stream);

/* Names of the main kernels one call launches, for matching measurements (kernel traces, counters)
 * to calls: the per-op times the pages compare (pytorch_block_sparse summary page, "Performance and
 * Memory Efficiency") are sums of these kernels. op: 0 bsr_linear_fwd, 1 bsr_linear_bwd_input,
 * 2 bsr_linear_bwd_weight (the bias-gradient kernels excluded), 3 bsr_linear_fwd_24; M rows. Writes a NUL-terminated,
 * comma-separated list (possibly empty) to buf[len]; BSR_ERR_INVALID_ARG for a NULL pattern or
 * buffer, an unknown op, M < 0 or a buffer too small. Host only, no device access. */
int32_t bsr_op_kernels(const bsr_pattern *p, int32_t op, int64_t M, char *buf, int32_t len);

/* Bytes of the per-GPU scratch array behind bsr_linear_bwd_weight_noalloc (32 MiB). */
#define BSR_NOALLOC_SCRATCH_BYTES (32u << 20)

/* Weight gradient exactly as bsr_linear_bwd_weight (same kernels, same result bit for bit), for
 * callers that cannot allocate device memory or pass a workspace: code under HIP graph capture,
 * tight serving or training loops, harnesses that forbid allocation. The scratch space (fp32
 * split-M partial sums of the kept blocks and of the bias) is a fixed array of
 * BSR_NOALLOC_SCRATCH_BYTES in the library's code object, one per GPU, created when the
 * library's kernels are loaded on that GPU and held until the process ends; the call makes no
 * allocation. Limits and sharing:
 *   - a call whose scratch need (bsr_linear_bwd_weight_workspace(p, M)) exceeds
 *     BSR_NOALLOC_SCRATCH_BYTES returns BSR_ERR_WORKSPACE_TOO_SMALL and enqueues nothing;
 *   - every call on one GPU uses that GPU's one array: calls whose work overlaps in time on one
 *     GPU (several streams, several threads) race and give wrong results; order them on one
 *     stream or synchronise between them. The array's contents between calls do not matter
 *     (each call writes every partial it reads).
 * Arguments and errors as for bsr_linear_bwd_weight. */
int32_t bsr_linear_bwd_weight_noalloc(const bsr_pattern *p, const bsr_bf16 *dY, const bsr_bf16 *X,
                                      int64_t M, bsr_bf16 *dV, bsr_bf16 *dbias, void *stream);

/* Static name of a status code ("BSR_OK", ...) of the calls above; the codes are this
 * library's own (the pages define no error interface). */
const char *bsr_status_string(int32_t status);

/* Detail of the last error on the calling thread ("" if none). Valid until the next call
 * on the same thread. */
const char *bsr_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BSR_LINEAR_H */
