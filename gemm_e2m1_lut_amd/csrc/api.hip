// api.hip -- the extern "C" entry points of libe2m1lut.so (declared in
// include/e2m1lut.h): host-side validation, then one asynchronous launch
// sequence on the caller's stream. Nothing here allocates, copies or
// synchronises; on a negative status nothing was launched.
#include <limits.h>

#include <mutex>

#include "e2m1lut.h"
#include "kernels.hpp"

namespace e2m1 {

int device_cu_count() {
    static int counts[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (counts[dev] == 0) {
        int c = 0;
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
            c = 256;
        counts[dev] = c;
    }
    return counts[dev];
}

}  // namespace e2m1

namespace {

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// a * b without signed overflow, for non-negative operands.
inline bool mul_ok(int64_t a, int64_t b) { return a == 0 || b <= INT64_MAX / a; }

inline int launch_status(hipError_t e) { return e == hipSuccess ? E2M1_OK : E2M1_ERR_LAUNCH; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

hipError_t fill_zero_bytes(void* dst, int64_t bytes, hipStream_t stream) {
    // Outputs are arrays of 2- or 4-byte elements: clear them as uint16.
    return e2m1::launch_fill_zero_u16(reinterpret_cast<uint16_t*>(dst), bytes / 2, stream);
}

// Workspace of mxfp4_moe_gemm_noalloc: one fixed array per GPU, held by the
// loaded code object until the process ends. In host code `scratch` names a
// host-side stand-in, not device memory, so it is never passed to a kernel or
// a copy: its device address is looked up once per device (with that device
// current, on the first call there) and that address is what the kernels get.
static __device__ __align__(256) uint8_t scratch[E2M1_MOE_NOALLOC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_status[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// Device address of the current device's `scratch` array.
hipError_t scratch_address(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        g_scratch_status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_status[dev] == hipSuccess ? p : nullptr;
    });
    if (g_scratch_status[dev] != hipSuccess) return g_scratch_status[dev];
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

int e2m1_abi_version(void) { return E2M1LUT_ABI_VERSION; }

const char* e2m1_strerror(int status) {
    switch (status) {
        case E2M1_OK: return "ok";
        case E2M1_ERR_NULL: return "a required pointer is NULL";
        case E2M1_ERR_SHAPE: return "invalid extent: negative, too large, or breaking a divisibility rule";
        case E2M1_ERR_ALIGN: return "a pointer is not aligned as the kernel's loads require";
        case E2M1_ERR_DTYPE: return "unknown output dtype code";
        case E2M1_ERR_WORKSPACE: return "workspace missing or smaller than the entry point's *_workspace_size()";
        case E2M1_ERR_LAUNCH: return "the HIP runtime reported an error at kernel launch";
        default: return "unknown status";
    }
}

int dequant_decode(const uint8_t* packed, const uint8_t* scale_e8m0, uint16_t* out_bf16,
                   int64_t rows, int64_t k, void* stream) {
    if (rows < 0 || k < 0 || k % 32 != 0 || !mul_ok(rows, k)) return E2M1_ERR_SHAPE;
    if (rows == 0 || k == 0) return E2M1_OK;
    if (!packed || !scale_e8m0 || !out_bf16) return E2M1_ERR_NULL;
    if (!aligned(packed, 16) || !aligned(out_bf16, 16)) return E2M1_ERR_ALIGN;
    return launch_status(e2m1::launch_decode(packed, scale_e8m0, out_bf16, rows * (k / 32),
                                             as_stream(stream)));
}

int dequant_gemv(const uint8_t* packed, const uint8_t* scale_e8m0, const uint16_t* x_bf16,
                 void* y, int y_dtype, int64_t batch, int64_t n, int64_t k, void* stream) {
    if (y_dtype != E2M1_DTYPE_F32 && y_dtype != E2M1_DTYPE_BF16) return E2M1_ERR_DTYPE;
    if (batch < 1 || batch > E2M1_GEMV_MAX_BATCH || n < 0 || k < 0 || k % 32 != 0 ||
        n > INT_MAX || k / 32 > INT_MAX / 64 || !mul_ok(n, k))
        return E2M1_ERR_SHAPE;
    if (n == 0) return E2M1_OK;
    const int64_t esize = y_dtype == E2M1_DTYPE_F32 ? 4 : 2;
    if (!y) return E2M1_ERR_NULL;
    if (!aligned(y, (uintptr_t)esize)) return E2M1_ERR_ALIGN;
    if (k == 0) return launch_status(fill_zero_bytes(y, batch * n * esize, as_stream(stream)));
    if (!packed || !scale_e8m0 || !x_bf16) return E2M1_ERR_NULL;
    if (!aligned(packed, 16) || !aligned(x_bf16, 16)) return E2M1_ERR_ALIGN;
    return launch_status(e2m1::launch_gemv(packed, scale_e8m0, x_bf16, y, y_dtype == E2M1_DTYPE_BF16,
                                           (int)batch, n, k, as_stream(stream)));
}

static_assert(E2M1_GEMV_MAX_GROUPS == e2m1::kGemvGroupMax, "group limit of the header and the kernels");

int dequant_gemv_grouped(int count, const uint8_t* const* packed, const uint8_t* const* scale_e8m0,
                         const uint16_t* const* x_bf16, void* const* y, const int64_t* n, const int64_t* k,
                         int y_dtype, void* stream) {
    if (y_dtype != E2M1_DTYPE_F32 && y_dtype != E2M1_DTYPE_BF16) return E2M1_ERR_DTYPE;
    if (count < 0 || count > E2M1_GEMV_MAX_GROUPS) return E2M1_ERR_SHAPE;
    if (count == 0) return E2M1_OK;
    if (!packed || !scale_e8m0 || !x_bf16 || !y || !n || !k) return E2M1_ERR_NULL;
    const int64_t esize = y_dtype == E2M1_DTYPE_F32 ? 4 : 2;
    for (int g = 0; g < count; ++g) {   // everything checked before the first launch
        if (n[g] < 0 || k[g] < 0 || k[g] % 32 != 0 || n[g] > INT_MAX || k[g] / 32 > INT_MAX / 64 ||
            !mul_ok(n[g], k[g]))
            return E2M1_ERR_SHAPE;
        if (n[g] == 0) continue;
        if (!y[g]) return E2M1_ERR_NULL;
        if (!aligned(y[g], (uintptr_t)esize)) return E2M1_ERR_ALIGN;
        if (k[g] == 0) continue;
        if (!packed[g] || !scale_e8m0[g] || !x_bf16[g]) return E2M1_ERR_NULL;
        if (!aligned(packed[g], 16) || !aligned(x_bf16[g], 16)) return E2M1_ERR_ALIGN;
    }
    e2m1::GemvMatrix mats[E2M1_GEMV_MAX_GROUPS];
    int m = 0;
    for (int g = 0; g < count; ++g) {
        if (n[g] == 0) continue;
        if (k[g] == 0) {
            const hipError_t err = fill_zero_bytes(y[g], n[g] * esize, as_stream(stream));
            if (err != hipSuccess) return launch_status(err);
            continue;
        }
        mats[m++] = e2m1::GemvMatrix{packed[g], scale_e8m0[g], x_bf16[g], y[g], n[g], k[g]};
    }
    if (m == 0) return E2M1_OK;
    return launch_status(e2m1::launch_gemv_group(mats, m, y_dtype == E2M1_DTYPE_BF16, as_stream(stream)));
}

int dequant_gemm(const uint8_t* packed, const uint8_t* scale_e8m0, const uint16_t* x_bf16, void* y,
                 int y_dtype, int64_t m, int64_t n, int64_t k, void* stream) {
    if (y_dtype != E2M1_DTYPE_F32 && y_dtype != E2M1_DTYPE_BF16) return E2M1_ERR_DTYPE;
    if (m < 0 || n < 0 || k < 0 || k % 32 != 0 || m > INT_MAX || n > INT_MAX || k > E2M1_GEMM_MAX_K ||
        !mul_ok(m, k) || !mul_ok(n, k) || !mul_ok(m, n) || ((n + 127) / 128) * ((m + 127) / 128) > INT_MAX)
        return E2M1_ERR_SHAPE;
    if (m == 0 || n == 0) return E2M1_OK;
    const int64_t esize = y_dtype == E2M1_DTYPE_F32 ? 4 : 2;
    if (!y) return E2M1_ERR_NULL;
    if (!aligned(y, (uintptr_t)esize)) return E2M1_ERR_ALIGN;
    if (k == 0) return launch_status(fill_zero_bytes(y, m * n * esize, as_stream(stream)));
    if (!packed || !scale_e8m0 || !x_bf16) return E2M1_ERR_NULL;
    if (!aligned(packed, 16) || !aligned(x_bf16, 16)) return E2M1_ERR_ALIGN;
    return launch_status(e2m1::launch_gemm(packed, scale_e8m0, x_bf16, y, y_dtype == E2M1_DTYPE_BF16, m, n, k,
                                           as_stream(stream)));
}

int nm_spmm(const uint16_t* values, const uint32_t* meta, const uint16_t* x_bf16, void* y, int y_dtype,
            int64_t batch, int64_t rows, int64_t k, int n_keep, int m_group, void* stream) {
    if (y_dtype != E2M1_DTYPE_F32 && y_dtype != E2M1_DTYPE_BF16) return E2M1_ERR_DTYPE;
    if (batch < 1 || batch > 16 || rows < 0 || k < 0 || m_group < 1 || m_group > 16 || n_keep < 1 ||
        n_keep > m_group || k % m_group != 0 || rows > INT_MAX || k > INT_MAX / 16 || !mul_ok(rows, k))
        return E2M1_ERR_SHAPE;
    if (rows == 0) return E2M1_OK;
    const int64_t esize = y_dtype == E2M1_DTYPE_F32 ? 4 : 2;
    if (!y) return E2M1_ERR_NULL;
    if (!aligned(y, (uintptr_t)esize)) return E2M1_ERR_ALIGN;
    if (k == 0) return launch_status(fill_zero_bytes(y, batch * rows * esize, as_stream(stream)));
    if (!values || !meta || !x_bf16) return E2M1_ERR_NULL;
    if (!aligned(values, 2) || !aligned(meta, 4) || !aligned(x_bf16, 2)) return E2M1_ERR_ALIGN;
    return launch_status(e2m1::launch_nm_spmm(values, meta, x_bf16, y, y_dtype == E2M1_DTYPE_BF16, batch, rows, k,
                                              n_keep, m_group, as_stream(stream)));
}

int mxfp4_quantize(const uint16_t* x_bf16, uint8_t* packed, uint8_t* scale_e8m0, int64_t rows,
                   int64_t k, void* stream) {
    if (rows < 0 || k < 0 || k % 32 != 0 || !mul_ok(rows, k)) return E2M1_ERR_SHAPE;
    if (rows == 0 || k == 0) return E2M1_OK;
    if (!x_bf16 || !packed || !scale_e8m0) return E2M1_ERR_NULL;
    if (!aligned(x_bf16, 16) || !aligned(packed, 8)) return E2M1_ERR_ALIGN;
    return launch_status(e2m1::launch_mxfp4_quantize(x_bf16, packed, scale_e8m0, rows * (k / 32),
                                                     as_stream(stream)));
}

int nvfp4_quantize(const uint16_t* x_bf16, const float* global_scale, uint8_t* packed,
                   uint8_t* block_scale_e4m3, int64_t rows, int64_t k, void* stream) {
    if (rows < 0 || k < 0 || k % 16 != 0 || !mul_ok(rows, k)) return E2M1_ERR_SHAPE;
    if (rows == 0 || k == 0) return E2M1_OK;
    if (!x_bf16 || !global_scale || !packed || !block_scale_e4m3) return E2M1_ERR_NULL;
    if (!aligned(x_bf16, 16) || !aligned(packed, 8) || !aligned(global_scale, 4)) return E2M1_ERR_ALIGN;
    return launch_status(e2m1::launch_nvfp4_quantize(x_bf16, global_scale, packed, block_scale_e4m3,
                                                     rows * (k / 16), as_stream(stream)));
}

int ternary_gemv(const uint32_t* packed, const float* row_scale, const float* x, float* y,
                 int64_t n, int64_t k, void* stream) {
    if (n < 0 || k < 0 || k % 16 != 0 || n > INT_MAX || k / 16 > INT_MAX / 64 || !mul_ok(n, k))
        return E2M1_ERR_SHAPE;
    if (n == 0) return E2M1_OK;
    if (!y) return E2M1_ERR_NULL;
    if (!aligned(y, 4)) return E2M1_ERR_ALIGN;
    if (k == 0) return launch_status(fill_zero_bytes(y, n * 4, as_stream(stream)));
    if (!packed || !row_scale || !x) return E2M1_ERR_NULL;
    if (!aligned(packed, 4) || !aligned(x, 4) || !aligned(row_scale, 4)) return E2M1_ERR_ALIGN;
    return launch_status(e2m1::launch_ternary(packed, row_scale, x, y, n, k, as_stream(stream)));
}

static bool ternary_gemm_shape_ok(int64_t batch, int64_t n, int64_t k) {
    return batch >= 1 && batch <= E2M1_TERNARY_MAX_BATCH && n >= 0 && k >= 0 && k % 16 == 0 && n <= INT_MAX &&
           k / 16 <= INT_MAX / 64 && mul_ok(n, k) && mul_ok(batch * 4, k) && mul_ok(batch * 4, n);
}

size_t ternary_gemm_workspace_size(int64_t batch, int64_t n, int64_t k) {
    if (!ternary_gemm_shape_ok(batch, n, k)) return SIZE_MAX;
    return n == 0 ? 0 : e2m1::ternary_gemm_workspace_bytes(batch, k);
}

int ternary_gemm(const uint32_t* packed, const float* row_scale, const float* x, float* y, void* workspace,
                 size_t workspace_bytes, int64_t batch, int64_t n, int64_t k, void* stream) {
    if (!ternary_gemm_shape_ok(batch, n, k)) return E2M1_ERR_SHAPE;
    if (n == 0) return E2M1_OK;
    if (!y) return E2M1_ERR_NULL;
    if (!aligned(y, 4)) return E2M1_ERR_ALIGN;
    if (k == 0) return launch_status(fill_zero_bytes(y, batch * n * 4, as_stream(stream)));
    if (!packed || !row_scale || !x) return E2M1_ERR_NULL;
    if (!aligned(packed, 4) || !aligned(x, 4) || !aligned(row_scale, 4)) return E2M1_ERR_ALIGN;
    const size_t need = e2m1::ternary_gemm_workspace_bytes(batch, k);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return E2M1_ERR_WORKSPACE;
        if (!aligned(workspace, 256)) return E2M1_ERR_ALIGN;
    }
    return launch_status(
        e2m1::launch_ternary_gemm(packed, row_scale, x, y, batch, n, k, workspace, as_stream(stream)));
}

int ternary_wl_gemv(const uint32_t* const packed[4], const float* scale, const float* x_re,
                    const float* x_im, float* y_re, float* y_im, int64_t n, int64_t k, void* stream) {
    if (n < 0 || k < 0 || k % 16 != 0 || n > INT_MAX || k / 16 > INT_MAX / 64 || !mul_ok(n, k) ||
        !mul_ok(n, 4))
        return E2M1_ERR_SHAPE;
    if (n == 0) return E2M1_OK;
    if (!y_re || !y_im) return E2M1_ERR_NULL;
    if (!aligned(y_re, 4) || !aligned(y_im, 4)) return E2M1_ERR_ALIGN;
    if (k == 0) {
        hipError_t e = fill_zero_bytes(y_re, n * 4, as_stream(stream));
        if (e == hipSuccess) e = fill_zero_bytes(y_im, n * 4, as_stream(stream));
        return launch_status(e);
    }
    if (!packed || !scale || !x_re || !x_im) return E2M1_ERR_NULL;
    for (int m = 0; m < 4; ++m) {
        if (!packed[m]) return E2M1_ERR_NULL;
        if (!aligned(packed[m], 4)) return E2M1_ERR_ALIGN;
    }
    if (!aligned(scale, 4) || !aligned(x_re, 4) || !aligned(x_im, 4)) return E2M1_ERR_ALIGN;
    return launch_status(e2m1::launch_ternary_wl(packed, scale, x_re, x_im, y_re, y_im, n, k,
                                                 as_stream(stream)));
}

int nvfp4_embedding_gather(const uint8_t* table, const uint8_t* block_scale_e4m3,
                           const float* global_scale, const int64_t* ids, uint16_t* out_bf16,
                           int64_t vocab, int64_t hidden, int64_t num_tokens, int32_t* err_flag,
                           void* stream) {
    if (vocab < 0 || hidden < 0 || num_tokens < 0 || hidden % 16 != 0 || !mul_ok(vocab, hidden) ||
        !mul_ok(num_tokens, hidden))
        return E2M1_ERR_SHAPE;
    if (num_tokens == 0 || hidden == 0) return E2M1_OK;
    if (!ids || !out_bf16 || !global_scale) return E2M1_ERR_NULL;
    if (vocab > 0 && (!table || !block_scale_e4m3)) return E2M1_ERR_NULL;
    if (!aligned(table, 8) || !aligned(out_bf16, 16) || !aligned(ids, 8) || !aligned(global_scale, 4) ||
        !aligned(err_flag, 4))
        return E2M1_ERR_ALIGN;
    return launch_status(e2m1::launch_nvfp4_gather(table, block_scale_e4m3, global_scale, ids,
                                                   out_bf16, vocab, hidden, num_tokens, err_flag,
                                                   as_stream(stream)));
}

size_t mxfp4_moe_workspace_size(int64_t tokens, int64_t hidden, int64_t inter, int64_t experts,
                                int64_t topk) {
    if (tokens < 0 || hidden < 0 || inter < 0 || experts < 1 || topk < 1 || hidden % 32 != 0 ||
        inter % 32 != 0 || !mul_ok(tokens, topk) || tokens * topk > INT_MAX)
        return (size_t)-1;
    if (tokens == 0 || hidden == 0) return 0;
    return e2m1::moe_workspace_bytes(tokens, hidden, inter, experts, topk);
}

int mxfp4_moe_gemm(const uint16_t* x, const uint8_t* w13, const uint8_t* w13_scale,
                   const uint8_t* w2, const uint8_t* w2_scale, const int32_t* topk_ids,
                   const float* topk_weights, uint16_t* out, void* workspace,
                   size_t workspace_bytes, int64_t tokens, int64_t hidden, int64_t inter,
                   int64_t experts, int64_t topk, void* stream) {
    const size_t need = mxfp4_moe_workspace_size(tokens, hidden, inter, experts, topk);
    if (need == (size_t)-1 || experts > E2M1_MOE_MAX_EXPERTS || hidden > INT_MAX || inter > INT_MAX ||
        inter * hidden >= ((int64_t)1 << 31))   // each expert's W13 (and W2) below 2 GiB: 32-bit offsets
        return E2M1_ERR_SHAPE;
    if (tokens == 0 || hidden == 0) return E2M1_OK;
    if (!x || !out || !topk_ids || !topk_weights) return E2M1_ERR_NULL;
    if (inter == 0) return launch_status(fill_zero_bytes(out, tokens * hidden * 2, as_stream(stream)));
    if (!w13 || !w13_scale || !w2 || !w2_scale) return E2M1_ERR_NULL;
    if (!workspace || workspace_bytes < need) return E2M1_ERR_WORKSPACE;
    if (!aligned(x, 16) || !aligned(w13, 16) || !aligned(w2, 16) || !aligned(out, 16) ||
        !aligned(workspace, 256) || !aligned(topk_ids, 4) || !aligned(topk_weights, 4))
        return E2M1_ERR_ALIGN;
    return launch_status(e2m1::launch_moe(x, w13, w13_scale, w2, w2_scale, topk_ids, topk_weights,
                                          out, workspace, tokens, hidden, inter, experts, topk,
                                          as_stream(stream)));
}

int mxfp4_moe_gemm_noalloc(const uint16_t* x, const uint8_t* w13, const uint8_t* w13_scale,
                           const uint8_t* w2, const uint8_t* w2_scale, const int32_t* topk_ids,
                           const float* topk_weights, uint16_t* out, int64_t tokens,
                           int64_t hidden, int64_t inter, int64_t experts, int64_t topk,
                           void* stream) {
    const size_t need = mxfp4_moe_workspace_size(tokens, hidden, inter, experts, topk);
    if (need == (size_t)-1 || experts > E2M1_MOE_MAX_EXPERTS || hidden > INT_MAX || inter > INT_MAX)
        return E2M1_ERR_SHAPE;
    if (need > E2M1_MOE_NOALLOC_WORKSPACE_BYTES) return E2M1_ERR_WORKSPACE;
    if (tokens == 0 || hidden == 0) return E2M1_OK;
    void* ws = nullptr;
    if (scratch_address(&ws) != hipSuccess) return E2M1_ERR_LAUNCH;
    // the same validation and launches as the workspace entry point
    return mxfp4_moe_gemm(x, w13, w13_scale, w2, w2_scale, topk_ids, topk_weights, out, ws,
                          E2M1_MOE_NOALLOC_WORKSPACE_BYTES, tokens, hidden, inter, experts, topk, stream);
}

}  // extern "C"
