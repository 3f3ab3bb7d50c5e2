// ternary.hip -- 2-bit ternary GEMV (ternary_gemv).
//
// Method: FairyFuse blog post, section "三元 GEMV 的乘法消除原理": 16 weights
// per 32-bit word; weight j of word w multiplies x[16w + j]; bit 2j+1 set
// adds x, bit 2j set subtracts x, neither contributes nothing; the per-row
// scale is the only multiply and is applied once, after the row sum.
//
// gfx950 design. The page's CPU kernel extracts +1/-1 lane masks with BMI2
// pext so that AVX-512 masked adds can use them; a GPU has no pext, but it
// does not need one: each lane owns fixed 64-column chunks of K (one 16-byte
// load = four words), keeps those 64 activations in registers for the whole
// kernel (staged once per workgroup through LDS), and tests the two bits of
// each field directly to add, subtract or skip. Lanes cover a row in groups
// (64 lanes for K >= 4096, fewer for short rows); the row total comes from a
// DPP / shuffle reduction and is multiplied by the row scale once.
#include "device.hpp"
#include "kernels.hpp"

namespace e2m1 {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;

// Add / subtract / skip for the 16 fields of one word against 16 activations.
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

// Fast path: K % 64 == 0, rows 16-byte aligned, K <= 64 * G * CPL.
template <int G, int CPL>
__global__ __launch_bounds__(kThreads) void ternary_kernel(const uint32_t* __restrict__ packed,
                                                           const float* __restrict__ row_scale,
                                                           const float* __restrict__ x,
                                                           float* __restrict__ y, int n, int kq) {
    extern __shared__ float4 xs4[];   // kq * 16 float4 = all of x
    constexpr int kRowsPerWave = kWave / G;
    const int lane = threadIdx.x & (kWave - 1);
    const int gl = lane & (G - 1);
    const int grp = lane / G;
    const int wave = blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    const int row_stride = gridDim.x * kWavesPerBlock * kRowsPerWave;
    const uint4* pk = reinterpret_cast<const uint4*>(packed);

    for (int i = threadIdx.x; i < kq * 16; i += kThreads) xs4[i] = reinterpret_cast<const float4*>(x)[i];
    __syncthreads();
    float xr[CPL][64];
#pragma unroll
    for (int ci = 0; ci < CPL; ++ci) {
        const int c = gl + G * ci;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const float4 v = (c < kq) ? xs4[c * 16 + q] : make_float4(0.f, 0.f, 0.f, 0.f);
            xr[ci][4 * q + 0] = v.x;
            xr[ci][4 * q + 1] = v.y;
            xr[ci][4 * q + 2] = v.z;
            xr[ci][4 * q + 3] = v.w;
        }
    }

    for (int base = wave * kRowsPerWave; base < n; base += row_stride) {
        const int row = base + grp;
        float acc = 0.f;
#pragma unroll
        for (int ci = 0; ci < CPL; ++ci) {
            const int c = gl + G * ci;
            if (row < n && c < kq) {
                const uint4 w = load_nt16(pk + (int64_t)row * kq + c);
                acc = ternary_word(w.x, xr[ci] + 0, acc);
                acc = ternary_word(w.y, xr[ci] + 16, acc);
                acc = ternary_word(w.z, xr[ci] + 32, acc);
                acc = ternary_word(w.w, xr[ci] + 48, acc);
            }
        }
        acc = group_sum<G>(acc);
        if (gl == 0 && row < n) y[row] = row_scale[row] * acc;
    }
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

template <int G, int CPL>
hipError_t run_fast(const uint32_t* packed, const float* s, const float* x, float* y, int n,
                    int kq, hipStream_t stream) {
    auto kernel = ternary_kernel<G, CPL>;
    const size_t lds = (size_t)kq * 256;
    const int rows_per_block = kWavesPerBlock * (kWave / G);
    const int want = (n + rows_per_block - 1) / rows_per_block;
    static int cap = 0;
    if (cap == 0) cap = resident_blocks(kernel, (size_t)256 * G * CPL);
    const int grid = want < cap ? want : cap;
    kernel<<<grid, kThreads, lds, stream>>>(packed, s, x, y, n, kq);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ternary(const uint32_t* packed, const float* row_scale, const float* x, float* y,
                          int64_t n, int64_t k, hipStream_t stream) {
    const int nn = (int)n;
    const bool aligned = (reinterpret_cast<uintptr_t>(packed) & 15u) == 0 &&
                         (reinterpret_cast<uintptr_t>(x) & 15u) == 0 && k % 64 == 0;
    if (aligned && k <= 64 * 64 * 2) {
        const int kq = (int)(k / 64);
        if (kq <= 8) return run_fast<8, 1>(packed, row_scale, x, y, nn, kq, stream);
        if (kq <= 16) return run_fast<16, 1>(packed, row_scale, x, y, nn, kq, stream);
        if (kq <= 32) return run_fast<32, 1>(packed, row_scale, x, y, nn, kq, stream);
        if (kq <= 64) return run_fast<64, 1>(packed, row_scale, x, y, nn, kq, stream);
        return run_fast<64, 2>(packed, row_scale, x, y, nn, kq, stream);
    }
    const int want = (nn + kWavesPerBlock - 1) / kWavesPerBlock;
    static int cap = 0;
    if (cap == 0) cap = resident_blocks(ternary_generic_kernel, 0);
    const int grid = want < cap ? want : cap;
    ternary_generic_kernel<<<grid, kThreads, 0, stream>>>(packed, row_scale, x, y, nn, (int)(k / 16));
    return hipGetLastError();
}

}  // namespace e2m1
