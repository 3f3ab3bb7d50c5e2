// ternary.hip -- 2-bit ternary GEMV (ternary_gemv).
//
// Method: FairyFuse blog post, section "三元 GEMV 的乘法消除原理": 16 weights
// per 32-bit word; weight j of word w multiplies x[16w + j]; bit 2j+1 set
// adds x, bit 2j set subtracts x, neither contributes nothing; the per-row
// scale is the only multiply and is applied once, after the row sum.
//
// gfx950 design. The page's CPU kernel extracts +1/-1 lane masks with BMI2
// pext so that AVX-512 masked adds can use them; a GPU has no pext, and a
// per-field compare-and-select costs about six VALU operations per weight.
// With K % 64 == 0 and 16-byte aligned weights the GEMV is the batch-1 case
// of the small-batch ternary GEMM (ternary_batch.hip): weights decode to
// int8 four at a time with one v_perm_b32 and the int8 matrix cores sum them
// exactly against fixed-point digits of x. Other inputs use a one-wave-per-row
// kernel that adds, subtracts or skips each x directly, in fp32.
#include "device.hpp"
#include "kernels.hpp"

namespace e2m1 {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;

// Add / subtract / skip for the 16 fields of one word against 16 activations
// (the slower kernel for unaligned or ragged inputs).
__device__ __forceinline__ float ternary_word(uint32_t w, const float* xv, float acc) {
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int j = 0; j < 16; j += 2) {
        const uint32_t f0 = (w >> (2 * j)) & 3u;
        const uint32_t f1 = (w >> (2 * j + 2)) & 3u;
        a0 += (f0 == 2u) ? xv[j] : ((f0 == 1u) ? -xv[j] : 0.f);
        a1 += (f1 == 2u) ? xv[j + 1] : ((f1 == 1u) ? -xv[j + 1] : 0.f);
    }
    return acc + (a0 + a1);
}

// Any K % 16 == 0: one wave per row, lanes across words, x from memory.
__global__ __launch_bounds__(kThreads) void ternary_generic_kernel(
    const uint32_t* __restrict__ packed, const float* __restrict__ row_scale,
    const float* __restrict__ x, float* __restrict__ y, int n, int kw) {
    const int lane = threadIdx.x & (kWave - 1);
    const int nwaves = gridDim.x * kWavesPerBlock;
    for (int row = blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; row < n; row += nwaves) {
        float acc = 0.f;
        for (int c = lane; c < kw; c += kWave)
            acc = ternary_word(packed[(int64_t)row * kw + c], x + 16 * c, acc);
        acc = group_sum<kWave>(acc);
        if (lane == 0) y[row] = row_scale[row] * acc;
    }
}

template <typename Kernel>
int resident_blocks(Kernel kernel, size_t lds_bytes) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, lds_bytes) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    return per_cu * device_cu_count();
}

}  // namespace

hipError_t launch_ternary(const uint32_t* packed, const float* row_scale, const float* x, float* y,
                          int64_t n, int64_t k, hipStream_t stream) {
    // K % 64 == 0 with 16-byte aligned weights: the int8 matrix-core kernel at batch 1
    if (k % 64 == 0 && (reinterpret_cast<uintptr_t>(packed) & 15u) == 0)
        return launch_ternary_gemm(packed, row_scale, x, y, 1, n, k, nullptr, stream);   // batch 1: no workspace
    const int nn = (int)n;
    const int want = (nn + kWavesPerBlock - 1) / kWavesPerBlock;
    static int cap = 0;
    if (cap == 0) cap = resident_blocks(ternary_generic_kernel, 0);
    const int grid = want < cap ? want : cap;
    ternary_generic_kernel<<<grid, kThreads, 0, stream>>>(packed, row_scale, x, y, nn, (int)(k / 16));
    return hipGetLastError();
}

}  // namespace e2m1
