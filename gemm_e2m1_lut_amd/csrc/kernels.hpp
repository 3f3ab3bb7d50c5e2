// kernels.hpp -- internal launch functions of libe2m1lut.so (not part of the C ABI).
// Arguments are validated by the C entry points in api.hip before these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace e2m1 {

// Compute units of the current device (cached per device).
int device_cu_count();

hipError_t launch_fill_zero_u16(uint16_t* dst, int64_t count, hipStream_t stream);

hipError_t launch_decode(const uint8_t* packed, const uint8_t* scales, uint16_t* out,
                         int64_t nblocks, hipStream_t stream);

hipError_t launch_mxfp4_quantize(const uint16_t* x, uint8_t* packed, uint8_t* scales, int64_t nblocks,
                                 hipStream_t stream);

hipError_t launch_nvfp4_quantize(const uint16_t* x, const float* global_scale, uint8_t* packed,
                                 uint8_t* block_scale, int64_t nblocks, hipStream_t stream);

hipError_t launch_gemv(const uint8_t* packed, const uint8_t* scales, const uint16_t* x, void* y,
                       bool out_bf16, int batch, int64_t n, int64_t k, hipStream_t stream);

// One batch-1 product of a grouped launch (host-side descriptor).
struct GemvMatrix {
    const uint8_t* packed;
    const uint8_t* scales;
    const uint16_t* x;
    void* y;
    int64_t n, k;
};
constexpr int kGemvGroupMax = 64;   // E2M1_GEMV_MAX_GROUPS
// count <= kGemvGroupMax matrices with n >= 1 and k >= 32 (validated by the caller).
hipError_t launch_gemv_group(const GemvMatrix* mats, int count, bool out_bf16, hipStream_t stream);

hipError_t launch_gemm(const uint8_t* packed, const uint8_t* scales, const uint16_t* x, void* y, bool out_bf16,
                       int64_t m, int64_t n, int64_t k, hipStream_t stream);

hipError_t launch_nm_spmm(const uint16_t* values, const uint32_t* meta, const uint16_t* x, void* y, bool out_bf16,
                          int64_t batch, int64_t rows, int64_t k, int nn, int mm, hipStream_t stream);

hipError_t launch_ternary(const uint32_t* packed, const float* row_scale, const float* x, float* y,
                          int64_t n, int64_t k, hipStream_t stream);

// Device workspace launch_ternary_gemm uses for (batch, k); 0 where it takes the one-launch kernels.
size_t ternary_gemm_workspace_bytes(int64_t batch, int64_t k);
hipError_t launch_ternary_gemm(const uint32_t* packed, const float* row_scale, const float* x, float* y,
                               int64_t batch, int64_t n, int64_t k, void* workspace, hipStream_t stream);

hipError_t launch_ternary_wl(const uint32_t* const mats[4], const float* scale, const float* x_re,
                             const float* x_im, float* y_re, float* y_im, int64_t n, int64_t k,
                             hipStream_t stream);

hipError_t launch_nvfp4_gather(const uint8_t* table, const uint8_t* block_scale,
                               const float* global_scale, const int64_t* ids, uint16_t* out,
                               int64_t vocab, int64_t hidden, int64_t ntok, int32_t* err_flag,
                               hipStream_t stream);

size_t moe_workspace_bytes(int64_t tokens, int64_t hidden, int64_t inter, int64_t experts,
                           int64_t topk);

hipError_t launch_moe(const uint16_t* x, const uint8_t* w13, const uint8_t* w13s,
                      const uint8_t* w2, const uint8_t* w2s, const int32_t* ids,
                      const float* weights, uint16_t* out, void* workspace, int64_t tokens,
                      int64_t hidden, int64_t inter, int64_t experts, int64_t topk,
                      hipStream_t stream);

}  // namespace e2m1
