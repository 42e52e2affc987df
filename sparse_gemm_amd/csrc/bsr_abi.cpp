// bsr_abi.cpp -- the extern "C" entry points: argument checks, pattern life cycle, dispatch.
// Nothing is enqueued before every argument has been checked; no C++ exception escapes.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <utility>
#include <vector>

#include "bsr_convert_internal.hpp"
#include "bsr_fp8_internal.hpp"
#include "bsr_rebuild_internal.hpp"
#include "bsr_sparse24_internal.hpp"

namespace bsr {

namespace {

bool aligned16(const void *ptr) { return ((uintptr_t)ptr & 15u) == 0; }

int32_t check_shape(int32_t N, int32_t K, int32_t b) {
    if (b != 32 && b != 64) return fail(BSR_ERR_UNSUPPORTED, "block size must be 32 or 64, got " + std::to_string(b));
    if (N <= 0 || K <= 0) return fail(BSR_ERR_INVALID_ARG, "N and K must be positive");
    if (N % b || K % b) return fail(BSR_ERR_INVALID_ARG, "N and K must be multiples of the block size");
    return BSR_OK;
}

// Copies every metadata array to the current device in one allocation.
int32_t upload(bsr_pattern &p) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(BSR_ERR_HIP, "hipGetDevice failed (no usable GPU?)");
    struct Part {
        const std::vector<int32_t> *v;
        const int32_t **dst;
    };
    DeviceMeta &d = p.dev;
    std::vector<Part> parts = {
        {&p.row_ptr, &d.row_ptr}, {&p.col_idx, &d.col_idx}, {&p.col_ptr, &d.col_ptr},
        {&p.row_idx, &d.row_idx}, {&p.perm, &d.perm},       {&p.small_m_rows, &d.small_m_rows},
        {&p.dw.items, &d.dw_items},         {&p.small_m_work, &d.small_m_work},
        {&p.wdw.items, &d.wdw_items},       {&p.wdw.compact, &d.wdw_compact},
    };
    for (int k = 0; k < kGemmVariants; ++k) {
        for (auto sd : {std::make_pair(&p.fwd[k], &d.fwd[k]), std::make_pair(&p.bwd[k], &d.bwd[k])}) {
            parts.push_back({&sd.first->order, &sd.second->order});
            parts.push_back({&sd.first->sub_ptr, &sd.second->sub_ptr});
            parts.push_back({&sd.first->out, &sd.second->out});
            parts.push_back({&sd.first->rec, &sd.second->rec});
        }
    }
    for (auto sd : {std::make_pair(&p.wide_fwd, &d.wide_fwd), std::make_pair(&p.wide_bwd, &d.wide_bwd)}) {
        parts.push_back({&sd.first->order, &sd.second->order});
        parts.push_back({&sd.first->sub_ptr, &sd.second->sub_ptr});
        parts.push_back({&sd.first->out, &sd.second->out});
        parts.push_back({&sd.first->rec, &sd.second->rec});
        parts.push_back({&sd.first->flags, &sd.second->flags});
    }
    size_t total = 0;
    for (const Part &q : parts) total += (q.v->size() * sizeof(int32_t) + 255) & ~size_t(255);
    if (total == 0) total = 256;
    std::vector<char> host(total, 0);
    size_t off = 0;
    std::vector<size_t> offs;
    for (const Part &q : parts) {
        offs.push_back(off);
        if (!q.v->empty()) std::memcpy(host.data() + off, q.v->data(), q.v->size() * sizeof(int32_t));
        off += (q.v->size() * sizeof(int32_t) + 255) & ~size_t(255);
    }
    void *base = nullptr;
    hipError_t e = hipMalloc(&base, total);
    if (e == hipErrorOutOfMemory) return fail(BSR_ERR_OUT_OF_MEMORY, "hipMalloc of pattern metadata failed");
    if (e != hipSuccess) return fail(BSR_ERR_HIP, std::string("hipMalloc: ") + hipGetErrorString(e));
    e = hipMemcpy(base, host.data(), total, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        (void)hipFree(base);
        return fail(BSR_ERR_HIP, std::string("hipMemcpy: ") + hipGetErrorString(e));
    }
    for (size_t k = 0; k < parts.size(); ++k)
        *parts[k].dst = reinterpret_cast<const int32_t *>(static_cast<char *>(base) + offs[k]);
    d.base = base;
    d.bytes = total;
    d.device = dev;
    p.uploaded = true;
    return BSR_OK;
}

int32_t finish_create(bsr_pattern *p, int32_t upload_flag, bsr_pattern **out) {
    if (p->nnzb > kMaxNnzb) {
        delete p;
        return fail(BSR_ERR_INVALID_ARG, "more than " + std::to_string(kMaxNnzb) + " kept blocks");
    }
    try {
        build_pattern(*p);
    } catch (const std::bad_alloc &) {
        delete p;
        return fail(BSR_ERR_OUT_OF_MEMORY, "host allocation failed while building the pattern");
    }
    if (upload_flag) {
        int32_t st = upload(*p);
        if (st != BSR_OK) {
            delete p;
            return st;
        }
    }
    *out = p;
    return BSR_OK;
}

// Common checks of a compute call; device_ok: the call also takes device-built patterns.
int32_t check_call(const bsr_pattern *p, int64_t M, bool device_ok = false) {
    if (!p) return fail(BSR_ERR_INVALID_ARG, "pattern is NULL");
    if (!p->uploaded) return fail(BSR_ERR_NO_DEVICE_DATA, "pattern was created without upload");
    if (p->device_built && !device_ok)
        return fail(BSR_ERR_UNSUPPORTED, "a device-built pattern serves bsr_linear_fwd, bsr_linear_bwd_input and "
                                         "bsr_linear_bwd_weight(_noalloc) only");
    if (M < 0) return fail(BSR_ERR_INVALID_ARG, "M must be >= 0");
    if (M > (int64_t)INT32_MAX) return fail(BSR_ERR_INVALID_ARG, "M must fit in int32");
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return fail(BSR_ERR_HIP, "hipGetDevice failed");
    if (dev != p->dev.device)
        return fail(BSR_ERR_INVALID_ARG, "current device " + std::to_string(dev) + " differs from the pattern's device " +
                                             std::to_string(p->dev.device));
    return BSR_OK;
}

int32_t check_ptr(const void *ptr, const char *name, bool nullable = false) {
    if (!ptr) return nullable ? BSR_OK : fail(BSR_ERR_INVALID_ARG, std::string(name) + " is NULL");
    if (!aligned16(ptr)) return fail(BSR_ERR_MISALIGNED, std::string(name) + " is not 16-byte aligned");
    return BSR_OK;
}

// The streaming small-M kernel (up to four 16-row tiles per work-group) beats the panel GEMM up to
// 64 rows for b = 64 (decode weight 8 x 4096 -> 14336: 17 rows 36.8 -> 16.1 us, 32 rows 37.1 -> 19.2,
// 64 rows 37.4 -> 29.5; 96 rows 46.8 against 37.5) and up to 32 rows for b = 32 (BERT-base FFN-up
// weight: 6.2 -> 4.1-4.4 us; even at 48 rows, behind from 64).
int64_t small_m_max(const bsr_pattern &p) {
    int64_t small_max = p.b == 64 ? 4 * kSmallM : 2 * kSmallM;
    if (const char *f = std::getenv("BSR_SMALLM_MAX")) small_max = std::atoll(f);   // tuning knob
    return small_max;
}

}  // namespace

}  // namespace bsr

using namespace bsr;

#define BSR_TRY_BEGIN try {
#define BSR_TRY_END                                                             \
    }                                                                           \
    catch (const std::bad_alloc &) {                                            \
        return fail(BSR_ERR_OUT_OF_MEMORY, "host allocation failed");           \
    }                                                                           \
    catch (...) {                                                               \
        return fail(BSR_ERR_INVALID_ARG, "unexpected internal exception");      \
    }

#define BSR_CHECK(expr)             \
    do {                            \
        int32_t _st = (expr);       \
        if (_st != BSR_OK) return _st; \
    } while (0)

extern "C" {

int32_t bsr_abi_version(void) { return BSR_ABI_VERSION; }

int32_t bsr_pattern_create_from_mask(int32_t N, int32_t K, int32_t b, const uint8_t *mask, int32_t upload_flag,
                                     bsr_pattern **out) {
    BSR_TRY_BEGIN
    if (!out) return fail(BSR_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    BSR_CHECK(check_shape(N, K, b));
    if (!mask) return fail(BSR_ERR_INVALID_ARG, "mask is NULL");
    auto *p = new bsr_pattern();
    p->N = N;
    p->K = K;
    p->b = b;
    p->R = N / b;
    p->C = K / b;
    csr_from_mask(p->R, p->C, mask, p->row_ptr, p->col_idx);
    p->nnzb = (int32_t)p->col_idx.size();
    return finish_create(p, upload_flag, out);
    BSR_TRY_END
}

int32_t bsr_pattern_create_from_csr(int32_t N, int32_t K, int32_t b, int32_t nnzb, const int32_t *row_ptr,
                                    const int32_t *col_idx, int32_t upload_flag, bsr_pattern **out) {
    BSR_TRY_BEGIN
    if (!out) return fail(BSR_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    BSR_CHECK(check_shape(N, K, b));
    const int32_t R = N / b, C = K / b;
    if (const char *why = check_csr(R, C, nnzb, row_ptr, col_idx)) return fail(BSR_ERR_INVALID_ARG, why);
    auto *p = new bsr_pattern();
    p->N = N;
    p->K = K;
    p->b = b;
    p->R = R;
    p->C = C;
    p->nnzb = nnzb;
    p->row_ptr.assign(row_ptr, row_ptr + R + 1);
    p->col_idx.assign(col_idx, col_idx + nnzb);
    return finish_create(p, upload_flag, out);
    BSR_TRY_END
}

int32_t bsr_pattern_info(const bsr_pattern *p, int32_t *N, int32_t *K, int32_t *b, int32_t *nnzb) {
    if (!p) return fail(BSR_ERR_INVALID_ARG, "pattern is NULL");
    if (N) *N = p->N;
    if (K) *K = p->K;
    if (b) *b = p->b;
    if (nnzb) *nnzb = p->nnzb;
    return BSR_OK;
}

int32_t bsr_pattern_export(const bsr_pattern *p, int32_t *row_ptr, int32_t *col_idx, int32_t *col_ptr,
                           int32_t *row_idx, int32_t *perm) {
    if (!p) return fail(BSR_ERR_INVALID_ARG, "pattern is NULL");
    if (p->device_built)
        return fail(BSR_ERR_UNSUPPORTED, "a device-built pattern has no host metadata (bsr_pattern_device_arrays)");
    auto put = [](int32_t *dst, const std::vector<int32_t> &v) {
        if (dst && !v.empty()) std::memcpy(dst, v.data(), v.size() * sizeof(int32_t));
    };
    put(row_ptr, p->row_ptr);
    put(col_idx, p->col_idx);
    put(col_ptr, p->col_ptr);
    put(row_idx, p->row_idx);
    put(perm, p->perm);
    return BSR_OK;
}

void bsr_pattern_destroy(bsr_pattern *p) {
    if (!p) return;
    if (p->dev.base) (void)hipFree(p->dev.base);
    delete p;
}

int32_t bsr_linear_fwd(const bsr_pattern *p, const bsr_bf16 *X, int64_t M, const bsr_bf16 *V, const bsr_bf16 *bias,
                       bsr_bf16 *Y, void *stream) {
    BSR_TRY_BEGIN
    BSR_CHECK(check_call(p, M, true));
    BSR_CHECK(check_ptr(X, "X", M == 0));
    BSR_CHECK(check_ptr(V, "V", p->nnzb == 0));
    BSR_CHECK(check_ptr(bias, "bias", true));
    BSR_CHECK(check_ptr(Y, "Y", M == 0));
    if (M == 0) return BSR_OK;
    FwdArgs a{X, M, p->K, V, bias, Y, p->N};
    if (p->device_built) {
        // device-built: the streaming forward straight from the device CSR (natural row order)
        if (M <= kSmallM) return launch_small_m_fwd_csr(p->N, p->K, p->b, p->dev.row_ptr, p->dev.col_idx, p->nnzb, a, stream);
    } else if (M <= small_m_max(*p)) {
        return launch_small_m_fwd(*p, a, stream);
    }
    return launch_group_gemm(*p, false, a, stream);
    BSR_TRY_END
}

int32_t bsr_linear_bwd_input(const bsr_pattern *p, const bsr_bf16 *dY, int64_t M, const bsr_bf16 *V, bsr_bf16 *dX,
                             void *stream) {
    BSR_TRY_BEGIN
    BSR_CHECK(check_call(p, M, true));
    BSR_CHECK(check_ptr(dY, "dY", M == 0));
    BSR_CHECK(check_ptr(V, "V", p->nnzb == 0));
    BSR_CHECK(check_ptr(dX, "dX", M == 0));
    if (M == 0) return BSR_OK;
    FwdArgs a{dY, M, p->N, V, nullptr, dX, p->K};
    return launch_group_gemm(*p, true, a, stream);
    BSR_TRY_END
}

int32_t bsr_op_kernels(const bsr_pattern *p, int32_t op, int64_t M, char *buf, int32_t len) {
    BSR_TRY_BEGIN
    if (!p) return fail(BSR_ERR_INVALID_ARG, "pattern is NULL");
    if (op < 0 || op > 3)
        return fail(BSR_ERR_INVALID_ARG,
                    "op must be 0 (forward), 1 (input gradient), 2 (weight gradient) or 3 (2:4 forward)");
    if (M < 0) return fail(BSR_ERR_INVALID_ARG, "M must be >= 0");
    if (!buf || len <= 0) return fail(BSR_ERR_INVALID_ARG, "buf must hold at least one byte");
    const std::string names = kernels_of(*p, op, M, small_m_max(*p));
    if ((int64_t)names.size() + 1 > len) return fail(BSR_ERR_INVALID_ARG, "buf too small for the kernel names");
    std::memcpy(buf, names.c_str(), names.size() + 1);
    return BSR_OK;
    BSR_TRY_END
}

size_t bsr_linear_bwd_weight_workspace(const bsr_pattern *p, int64_t M) {
    if (!p || M < 0) return 0;
    return dw_workspace_bytes(*p, M);
}

int32_t bsr_linear_bwd_weight(const bsr_pattern *p, const bsr_bf16 *dY, const bsr_bf16 *X, int64_t M, bsr_bf16 *dV,
                              bsr_bf16 *dbias, void *workspace, size_t ws_bytes, void *stream) {
    BSR_TRY_BEGIN
    BSR_CHECK(check_call(p, M, true));
    BSR_CHECK(check_ptr(dY, "dY", M == 0));
    BSR_CHECK(check_ptr(X, "X", M == 0));
    BSR_CHECK(check_ptr(dV, "dV", p->nnzb == 0));
    BSR_CHECK(check_ptr(dbias, "dbias", true));
    const size_t need = dw_workspace_bytes(*p, M);
    if (need > 0) {
        if (ws_bytes < need)
            return fail(BSR_ERR_WORKSPACE_TOO_SMALL,
                        "workspace of " + std::to_string(ws_bytes) + " bytes, need " + std::to_string(need));
        BSR_CHECK(check_ptr(workspace, "workspace"));
    }
    DwArgs a{dY, X, M, dV, dbias, workspace, ws_bytes};
    return launch_dw(*p, a, stream);
    BSR_TRY_END
}

int32_t bsr_linear_bwd_weight_noalloc(const bsr_pattern *p, const bsr_bf16 *dY, const bsr_bf16 *X, int64_t M,
                                      bsr_bf16 *dV, bsr_bf16 *dbias, void *stream) {
    BSR_TRY_BEGIN
    BSR_CHECK(check_call(p, M, true));
    BSR_CHECK(check_ptr(dY, "dY", M == 0));
    BSR_CHECK(check_ptr(X, "X", M == 0));
    BSR_CHECK(check_ptr(dV, "dV", p->nnzb == 0));
    BSR_CHECK(check_ptr(dbias, "dbias", true));
    const size_t need = dw_workspace_bytes(*p, M);
    if (need > (size_t)BSR_NOALLOC_SCRATCH_BYTES)
        return fail(BSR_ERR_WORKSPACE_TOO_SMALL,
                    "this pattern and M need " + std::to_string(need) + " bytes of scratch, above the " +
                        std::to_string((size_t)BSR_NOALLOC_SCRATCH_BYTES) +
                        " of the allocation-free call; use bsr_linear_bwd_weight with a workspace");
    void *ws = nullptr;
    if (need > 0) BSR_CHECK(noalloc_scratch(&ws));
    DwArgs a{dY, X, M, dV, dbias, ws, need};
    return launch_dw(*p, a, stream);
    BSR_TRY_END
}

int32_t bsr_block_norms(int32_t N, int32_t K, int32_t b, const bsr_bf16 *W, int32_t kind, double *norms,
                        void *stream) {
    BSR_TRY_BEGIN
    BSR_CHECK(check_shape(N, K, b));
    if (kind != BSR_NORM_L1 && kind != BSR_NORM_L2_SQUARED) return fail(BSR_ERR_INVALID_ARG, "unknown norm kind");
    if (N / b >= 65536) return fail(BSR_ERR_INVALID_ARG, "N/b must be below 65536");
    BSR_CHECK(check_ptr(W, "W"));
    BSR_CHECK(check_ptr(norms, "norms"));
    return launch_block_norms(N, K, b, W, kind, norms, stream);
    BSR_TRY_END
}

int32_t bsr_mask_topk(int32_t R, int32_t C, const double *norms, int64_t keep, uint8_t *mask) {
    BSR_TRY_BEGIN
    if (R <= 0 || C <= 0) return fail(BSR_ERR_INVALID_ARG, "R and C must be positive");
    if (keep < 0 || keep > (int64_t)R * C) return fail(BSR_ERR_INVALID_ARG, "keep must lie in [0, R*C]");
    if (!norms || !mask) return fail(BSR_ERR_INVALID_ARG, "norms and mask must not be NULL");
    return mask_topk(R, C, norms, keep, mask);
    BSR_TRY_END
}

int32_t bsr_pattern_create_from_dense(int32_t N, int32_t K, int32_t b, const bsr_bf16 *W, int32_t kind,
                                      int64_t keep, void *stream, bsr_pattern **out) {
    BSR_TRY_BEGIN
    if (!out) return fail(BSR_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    BSR_CHECK(check_shape(N, K, b));
    const int32_t R = N / b, C = K / b;
    if (keep < 0 || keep > (int64_t)R * C) return fail(BSR_ERR_INVALID_ARG, "keep must lie in [0, R*C]");
    const size_t bytes = sizeof(double) * (size_t)R * (size_t)C;
    double *dnorms = nullptr;
    hipError_t e = hipMalloc(&dnorms, bytes);
    if (e == hipErrorOutOfMemory) return fail(BSR_ERR_OUT_OF_MEMORY, "hipMalloc of the block norms failed");
    if (e != hipSuccess) return fail(BSR_ERR_HIP, std::string("hipMalloc: ") + hipGetErrorString(e));
    std::vector<double> norms((size_t)R * C);
    int32_t st = bsr_block_norms(N, K, b, W, kind, dnorms, stream);
    if (st == BSR_OK) {
        hipStream_t hs = static_cast<hipStream_t>(stream);
        e = hipMemcpyAsync(norms.data(), dnorms, bytes, hipMemcpyDeviceToHost, hs);
        if (e == hipSuccess) e = hipStreamSynchronize(hs);
        if (e != hipSuccess) st = fail(BSR_ERR_HIP, std::string("copying the block norms: ") + hipGetErrorString(e));
    }
    (void)hipFree(dnorms);
    if (st != BSR_OK) return st;
    std::vector<uint8_t> mask((size_t)R * C);
    BSR_CHECK(mask_topk(R, C, norms.data(), keep, mask.data()));
    return bsr_pattern_create_from_mask(N, K, b, mask.data(), 1, out);
    BSR_TRY_END
}

int32_t bsr_dense_to_values(const bsr_pattern *p, const bsr_bf16 *W, bsr_bf16 *V, void *stream) {
    BSR_TRY_BEGIN
    BSR_CHECK(check_call(p, 0));
    BSR_CHECK(check_ptr(W, "W"));
    BSR_CHECK(check_ptr(V, "V", p->nnzb == 0));
    return launch_dense_to_values(*p, W, V, stream);
    BSR_TRY_END
}

int32_t bsr_values_to_dense(const bsr_pattern *p, const bsr_bf16 *V, bsr_bf16 *W, void *stream) {
    BSR_TRY_BEGIN
    BSR_CHECK(check_call(p, 0));
    BSR_CHECK(check_ptr(V, "V", p->nnzb == 0));
    BSR_CHECK(check_ptr(W, "W"));
    if (p->R >= 65536) return fail(BSR_ERR_INVALID_ARG, "N/b must be below 65536");
    return launch_values_to_dense(*p, V, W, stream);
    BSR_TRY_END
}

int32_t bsr_values_quantize_fp8(const bsr_pattern *p, const bsr_bf16 *V, uint8_t *V8, int32_t *se, void *stream) {
    BSR_TRY_BEGIN
    BSR_CHECK(check_call(p, 0));
    BSR_CHECK(check_ptr(V, "V", p->nnzb == 0));
    BSR_CHECK(check_ptr(V8, "V8", p->nnzb == 0));
    if (p->nnzb > 0 && (!se || ((uintptr_t)se & 3u)))
        return fail(se ? BSR_ERR_MISALIGNED : BSR_ERR_INVALID_ARG, "se must be a 4-byte aligned device pointer");
    return launch_quantize_fp8(*p, V, V8, se, stream);
    BSR_TRY_END
}

int32_t bsr_values_dequantize_fp8(const bsr_pattern *p, const uint8_t *V8, const int32_t *se, bsr_bf16 *V,
                                  void *stream) {
    BSR_TRY_BEGIN
    BSR_CHECK(check_call(p, 0));
    BSR_CHECK(check_ptr(V8, "V8", p->nnzb == 0));
    BSR_CHECK(check_ptr(V, "V", p->nnzb == 0));
    if (p->nnzb > 0 && (!se || ((uintptr_t)se & 3u)))
        return fail(se ? BSR_ERR_MISALIGNED : BSR_ERR_INVALID_ARG, "se must be a 4-byte aligned device pointer");
    return launch_dequantize_fp8(*p, V8, se, V, stream);
    BSR_TRY_END
}

int32_t bsr_linear_fwd_fp8(const bsr_pattern *p, const bsr_bf16 *X, int64_t M, const uint8_t *V8, const int32_t *se,
                           const bsr_bf16 *bias, bsr_bf16 *Y, void *stream) {
    BSR_TRY_BEGIN
    BSR_CHECK(check_call(p, M));
    BSR_CHECK(check_ptr(X, "X", M == 0));
    BSR_CHECK(check_ptr(V8, "V8", p->nnzb == 0));
    if (p->nnzb > 0 && (!se || ((uintptr_t)se & 3u)))
        return fail(se ? BSR_ERR_MISALIGNED : BSR_ERR_INVALID_ARG, "se must be a 4-byte aligned device pointer");
    BSR_CHECK(check_ptr(bias, "bias", true));
    BSR_CHECK(check_ptr(Y, "Y", M == 0));
    if (M >= (int64_t)1 << 20) return fail(BSR_ERR_INVALID_ARG, "the fp8 forward takes M below 2^20");
    if ((int64_t)16 * p->K * 2 > (int64_t)UINT32_MAX) return fail(BSR_ERR_INVALID_ARG, "rows of X too long");
    if (M == 0) return BSR_OK;
    return launch_fwd_fp8(*p, X, M, V8, se, bias, Y, stream);
    BSR_TRY_END
}

int32_t bsr_values_compress_24(const bsr_pattern *p, const bsr_bf16 *V, bsr_bf16 *Vc, uint16_t *meta, void *stream) {
    BSR_TRY_BEGIN
    BSR_CHECK(check_call(p, 0));
    BSR_CHECK(check_ptr(V, "V", p->nnzb == 0));
    BSR_CHECK(check_ptr(Vc, "Vc", p->nnzb == 0));
    BSR_CHECK(check_ptr(meta, "meta", p->nnzb == 0));
    return launch_compress_24(*p, V, Vc, meta, stream);
    BSR_TRY_END
}

int32_t bsr_values_decompress_24(const bsr_pattern *p, const bsr_bf16 *Vc, const uint16_t *meta, bsr_bf16 *V,
                                 void *stream) {
    BSR_TRY_BEGIN
    BSR_CHECK(check_call(p, 0));
    BSR_CHECK(check_ptr(Vc, "Vc", p->nnzb == 0));
    BSR_CHECK(check_ptr(meta, "meta", p->nnzb == 0));
    BSR_CHECK(check_ptr(V, "V", p->nnzb == 0));
    return launch_decompress_24(*p, Vc, meta, V, stream);
    BSR_TRY_END
}

int32_t bsr_linear_fwd_24(const bsr_pattern *p, const bsr_bf16 *X, int64_t M, const bsr_bf16 *Vc, const uint16_t *meta,
                          const bsr_bf16 *bias, bsr_bf16 *Y, void *stream) {
    BSR_TRY_BEGIN
    BSR_CHECK(check_call(p, M));
    BSR_CHECK(check_ptr(X, "X", M == 0));
    BSR_CHECK(check_ptr(Vc, "Vc", p->nnzb == 0));
    BSR_CHECK(check_ptr(meta, "meta", p->nnzb == 0));
    BSR_CHECK(check_ptr(bias, "bias", true));
    BSR_CHECK(check_ptr(Y, "Y", M == 0));
    if (M >= (int64_t)1 << 20) return fail(BSR_ERR_INVALID_ARG, "the 2:4 forward takes M below 2^20");
    if ((size_t)p->nnzb * p->b * p->b >= (size_t)0xFFFFFFF0u)
        return fail(BSR_ERR_INVALID_ARG, "compressed block values above 4 GiB");
    if (M == 0) return BSR_OK;
    // many rows over block rows kept in most panels: the wide tile on the compressed blocks
    if (use_wide(*p, false, M)) {
        const FwdArgs a{X, M, p->K, nullptr, bias, Y, p->N};
        return launch_wide_gemm_24(*p, a, Vc, meta, stream);
    }
    // many rows otherwise: the panel GEMM staging the compressed blocks as they are
    if (M > small_m_max(*p)) {
        const FwdArgs a{X, M, p->K, Vc, bias, Y, p->N};
        return launch_group_gemm(*p, false, a, stream, true, meta);
    }
    if ((int64_t)16 * p->K * 2 > (int64_t)UINT32_MAX) return fail(BSR_ERR_INVALID_ARG, "rows of X too long");
    return launch_fwd_24(*p, X, M, Vc, meta, bias, Y, stream);
    BSR_TRY_END
}

int32_t bsr_values_quantize_fp8_24(const bsr_pattern *p, const bsr_bf16 *Vc, uint8_t *Vc8, int32_t *se, void *stream) {
    BSR_TRY_BEGIN
    BSR_CHECK(check_call(p, 0));
    BSR_CHECK(check_ptr(Vc, "Vc", p->nnzb == 0));
    BSR_CHECK(check_ptr(Vc8, "Vc8", p->nnzb == 0));
    if (p->nnzb > 0 && (!se || ((uintptr_t)se & 3u)))
        return fail(se ? BSR_ERR_MISALIGNED : BSR_ERR_INVALID_ARG, "se must be a 4-byte aligned device pointer");
    return launch_quantize_fp8(*p, Vc, Vc8, se, stream, true);
    BSR_TRY_END
}

int32_t bsr_linear_fwd_fp8_24(const bsr_pattern *p, const bsr_bf16 *X, int64_t M, const uint8_t *Vc8, const int32_t *se,
                              const uint16_t *meta, const bsr_bf16 *bias, bsr_bf16 *Y, void *stream) {
    BSR_TRY_BEGIN
    BSR_CHECK(check_call(p, M));
    BSR_CHECK(check_ptr(X, "X", M == 0));
    BSR_CHECK(check_ptr(Vc8, "Vc8", p->nnzb == 0));
    if (p->nnzb > 0 && (!se || ((uintptr_t)se & 3u)))
        return fail(se ? BSR_ERR_MISALIGNED : BSR_ERR_INVALID_ARG, "se must be a 4-byte aligned device pointer");
    BSR_CHECK(check_ptr(meta, "meta", p->nnzb == 0));
    BSR_CHECK(check_ptr(bias, "bias", true));
    BSR_CHECK(check_ptr(Y, "Y", M == 0));
    if (M >= (int64_t)1 << 20) return fail(BSR_ERR_INVALID_ARG, "the 2:4 forward takes M below 2^20");
    if ((size_t)p->nnzb * p->b * p->b >= (size_t)0xFFFFFFF0u)
        return fail(BSR_ERR_INVALID_ARG, "compressed block values above 4 GiB");
    if ((int64_t)16 * p->K * 2 > (int64_t)UINT32_MAX) return fail(BSR_ERR_INVALID_ARG, "rows of X too long");
    if (M == 0) return BSR_OK;
    return launch_fwd_fp8_24(*p, X, M, Vc8, se, meta, bias, Y, stream);
    BSR_TRY_END
}

int32_t bsr_values_pack_24(const bsr_pattern *p, const bsr_bf16 *Vc, const uint16_t *meta, uint16_t *img, void *stream) {
    BSR_TRY_BEGIN
    BSR_CHECK(check_call(p, 0));
    BSR_CHECK(check_ptr(Vc, "Vc", p->nnzb == 0));
    BSR_CHECK(check_ptr(meta, "meta", p->nnzb == 0));
    BSR_CHECK(check_ptr(img, "img", p->nnzb == 0));
    return launch_pack_24(*p, Vc, meta, img, stream);
    BSR_TRY_END
}

int32_t bsr_linear_fwd_24_image(const bsr_pattern *p, const bsr_bf16 *X, int64_t M, const uint16_t *img,
                                const bsr_bf16 *bias, bsr_bf16 *Y, void *stream) {
    BSR_TRY_BEGIN
    BSR_CHECK(check_call(p, M));
    BSR_CHECK(check_ptr(X, "X", M == 0));
    BSR_CHECK(check_ptr(img, "img", p->nnzb == 0));
    BSR_CHECK(check_ptr(bias, "bias", true));
    BSR_CHECK(check_ptr(Y, "Y", M == 0));
    if (M == 0) return BSR_OK;
    FwdArgs a{X, M, p->K, img, bias, Y, p->N};
    return launch_group_gemm(*p, false, a, stream, true);
    BSR_TRY_END
}

int32_t bsr_linear_fwd_small_m_csr(int32_t N, int32_t K, int32_t b, const int32_t *row_ptr, const int32_t *col_idx,
                                   int32_t cap, const bsr_bf16 *X, int64_t M, const bsr_bf16 *V, const bsr_bf16 *bias,
                                   bsr_bf16 *Y, void *stream) {
    BSR_TRY_BEGIN
    BSR_CHECK(check_shape(N, K, b));
    if (M < 0 || M > kSmallM) return fail(BSR_ERR_INVALID_ARG, "M must lie in [0, 16]");
    if (cap < 0) return fail(BSR_ERR_INVALID_ARG, "cap must be >= 0");
    if ((size_t)cap * b * b * 2 > (size_t)UINT32_MAX) return fail(BSR_ERR_INVALID_ARG, "cap * b * b values above 4 GiB");
    if (!row_ptr || !col_idx || ((uintptr_t)row_ptr & 3u) || ((uintptr_t)col_idx & 3u))
        return fail(BSR_ERR_INVALID_ARG, "row_ptr and col_idx must be 4-byte aligned device pointers");
    BSR_CHECK(check_ptr(X, "X", M == 0));
    BSR_CHECK(check_ptr(V, "V", true));
    BSR_CHECK(check_ptr(bias, "bias", true));
    BSR_CHECK(check_ptr(Y, "Y", M == 0));
    if (M == 0) return BSR_OK;
    if (!V) return fail(BSR_ERR_INVALID_ARG, "V is NULL");
    FwdArgs a{X, M, K, V, bias, Y, N};
    return launch_small_m_fwd_csr(N, K, b, row_ptr, col_idx, cap, a, stream);
    BSR_TRY_END
}

size_t bsr_meta_rebuild_workspace(int32_t R, int32_t C) {
    if (R <= 0 || C <= 0) return 0;
    return rebuild_workspace_bytes(R, C);
}

int32_t bsr_meta_rebuild(int32_t R, int32_t C, const uint8_t *mask, int32_t *row_ptr, int32_t *col_idx,
                         int32_t *col_ptr, int32_t *row_idx, int32_t *perm, int32_t cap, int32_t *nnzb,
                         void *workspace, size_t ws_bytes, void *stream) {
    BSR_TRY_BEGIN
    if (R <= 0 || C <= 0) return fail(BSR_ERR_INVALID_ARG, "R and C must be positive");
    if ((int64_t)R * C >= (int64_t)INT32_MAX) return fail(BSR_ERR_INVALID_ARG, "R*C must be below 2^31");
    if (cap < 0) return fail(BSR_ERR_INVALID_ARG, "cap must be >= 0");
    if (!mask || !row_ptr || !col_ptr || !nnzb || !workspace)
        return fail(BSR_ERR_INVALID_ARG, "mask, row_ptr, col_ptr, nnzb and workspace must not be NULL");
    if (cap > 0 && (!col_idx || !row_idx || !perm))
        return fail(BSR_ERR_INVALID_ARG, "col_idx, row_idx and perm must not be NULL when cap > 0");
    for (const void *ptr : {(const void *)row_ptr, (const void *)col_idx, (const void *)col_ptr, (const void *)row_idx,
                            (const void *)perm, (const void *)nnzb, (const void *)workspace})
        if ((uintptr_t)ptr & 3u) return fail(BSR_ERR_MISALIGNED, "device pointers must be 4-byte aligned");
    const size_t need = rebuild_workspace_bytes(R, C);
    if (ws_bytes < need)
        return fail(BSR_ERR_WORKSPACE_TOO_SMALL,
                    "workspace of " + std::to_string(ws_bytes) + " bytes, need " + std::to_string(need));
    return launch_rebuild(R, C, mask, row_ptr, col_idx, col_ptr, row_idx, perm, cap, nnzb, workspace, stream);
    BSR_TRY_END
}

int32_t bsr_pattern_create_device(int32_t N, int32_t K, int32_t b, int32_t cap, bsr_pattern **out) {
    BSR_TRY_BEGIN
    if (!out) return fail(BSR_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    BSR_CHECK(check_shape(N, K, b));
    const int32_t R = N / b, C = K / b;
    if ((int64_t)R * C >= (int64_t)INT32_MAX) return fail(BSR_ERR_INVALID_ARG, "R*C must be below 2^31");
    if (cap < 1 || cap > kMaxNnzb || (int64_t)cap > (int64_t)R * C)
        return fail(BSR_ERR_INVALID_ARG, "cap must lie in [1, min(2^23 - 1, (N/b)*(K/b))]");
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(BSR_ERR_HIP, "hipGetDevice failed (no usable GPU?)");
    auto *p = new bsr_pattern();
    p->N = N;
    p->K = K;
    p->b = b;
    p->R = R;
    p->C = C;
    p->nnzb = cap;
    p->device_built = true;
    const GemmVariant v = gemm_variant(b, kDeviceVariant);
    const int32_t gf = (R + v.G - 1) / v.G, gb = (C + v.G - 1) / v.G;
    for (auto [s, n] : {std::make_pair(&p->fwd[kDeviceVariant], gf), std::make_pair(&p->bwd[kDeviceVariant], gb)}) {
        s->G = v.G;
        s->S = v.S;
        s->ngroups = n;
    }
    const int64_t TR = dw_tile_rows(b), TC = dw_tile_cols(b), capi = (int64_t)kDwWaves * dw_slots(b);
    const int64_t ntiles = ((R + TR - 1) / TR) * ((C + TC - 1) / TC);
    p->dw.n = (int)std::min<int64_t>(cap, ntiles * ((TR * TC + capi - 1) / capi));
    // one allocation, zeroed: before the first rebuild the pattern is empty (every row pointer,
    // sub-step pointer and live count 0)
    struct Part {
        size_t ints;
        const int32_t **dst;
    };
    DeviceMeta &d = p->dev;
    const Part parts[] = {
        {(size_t)R + 1, &d.row_ptr}, {(size_t)cap, &d.col_idx}, {(size_t)C + 1, &d.col_ptr}, {(size_t)cap, &d.row_idx},
        {(size_t)cap, &d.perm}, {1, &d.live_nnzb}, {1, &d.live_items},
        {(size_t)gf, &d.fwd[kDeviceVariant].order}, {(size_t)gf + 1, &d.fwd[kDeviceVariant].sub_ptr},
        {(size_t)gf * v.G, &d.fwd[kDeviceVariant].out}, {(size_t)cap * kRecInts, &d.fwd[kDeviceVariant].rec},
        {(size_t)gb, &d.bwd[kDeviceVariant].order}, {(size_t)gb + 1, &d.bwd[kDeviceVariant].sub_ptr},
        {(size_t)gb * v.G, &d.bwd[kDeviceVariant].out}, {(size_t)cap * kRecInts, &d.bwd[kDeviceVariant].rec},
        {(size_t)p->dw.n * kDwItemInts, &d.dw_items},
    };
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    size_t total = 0;
    for (const Part &q : parts) total += al(q.ints * sizeof(int32_t));
    const size_t sched_bytes = sched_scratch_bytes(R, C, b), rebuild_bytes = rebuild_workspace_bytes(R, C);
    total += al(sched_bytes) + al(rebuild_bytes);
    void *base = nullptr;
    hipError_t e = hipMalloc(&base, total);
    if (e != hipSuccess) {
        delete p;
        return fail(e == hipErrorOutOfMemory ? BSR_ERR_OUT_OF_MEMORY : BSR_ERR_HIP,
                    std::string("hipMalloc of a device-built pattern: ") + hipGetErrorString(e));
    }
    e = hipMemset(base, 0, total);
    if (e != hipSuccess) {
        (void)hipFree(base);
        delete p;
        return fail(BSR_ERR_HIP, std::string("hipMemset: ") + hipGetErrorString(e));
    }
    char *c = static_cast<char *>(base);
    for (const Part &q : parts) {
        *q.dst = reinterpret_cast<const int32_t *>(c);
        c += al(q.ints * sizeof(int32_t));
    }
    d.sched_scratch = c;
    c += al(sched_bytes);
    d.rebuild_ws = c;
    d.base = base;
    d.bytes = total;
    d.device = dev;
    p->uploaded = true;
    *out = p;
    return BSR_OK;
    BSR_TRY_END
}

int32_t bsr_pattern_rebuild(bsr_pattern *p, const uint8_t *mask, void *stream) {
    BSR_TRY_BEGIN
    BSR_CHECK(check_call(p, 0, true));
    if (!p->device_built) return fail(BSR_ERR_UNSUPPORTED, "pattern is not device-built (bsr_pattern_create_device)");
    if (!mask) return fail(BSR_ERR_INVALID_ARG, "mask is NULL");
    return launch_pattern_rebuild(*p, mask, stream);
    BSR_TRY_END
}

int32_t bsr_pattern_device_arrays(const bsr_pattern *p, const int32_t **row_ptr, const int32_t **col_idx,
                                  const int32_t **col_ptr, const int32_t **row_idx, const int32_t **perm,
                                  const int32_t **nnzb) {
    if (!p) return fail(BSR_ERR_INVALID_ARG, "pattern is NULL");
    if (!p->device_built) return fail(BSR_ERR_UNSUPPORTED, "pattern is not device-built (bsr_pattern_create_device)");
    if (row_ptr) *row_ptr = p->dev.row_ptr;
    if (col_idx) *col_idx = p->dev.col_idx;
    if (col_ptr) *col_ptr = p->dev.col_ptr;
    if (row_idx) *row_idx = p->dev.row_idx;
    if (perm) *perm = p->dev.perm;
    if (nnzb) *nnzb = p->dev.live_nnzb;
    return BSR_OK;
}

const char *bsr_status_string(int32_t status) {
    switch (status) {
        case BSR_OK: return "BSR_OK";
        case BSR_ERR_INVALID_ARG: return "BSR_ERR_INVALID_ARG";
        case BSR_ERR_UNSUPPORTED: return "BSR_ERR_UNSUPPORTED";
        case BSR_ERR_MISALIGNED: return "BSR_ERR_MISALIGNED";
        case BSR_ERR_WORKSPACE_TOO_SMALL: return "BSR_ERR_WORKSPACE_TOO_SMALL";
        case BSR_ERR_HIP: return "BSR_ERR_HIP";
        case BSR_ERR_OUT_OF_MEMORY: return "BSR_ERR_OUT_OF_MEMORY";
        case BSR_ERR_NO_DEVICE_DATA: return "BSR_ERR_NO_DEVICE_DATA";
        default: return "BSR_ERR_UNKNOWN";
    }
}

const char *bsr_last_error(void) { return last_error(); }

}  // extern "C"
