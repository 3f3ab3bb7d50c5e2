// gemv.hip -- MXFP4 dequant-GEMV / small-batch GEMM (dequant_gemv).
//
// y[b, n] = sum_k W[n, k] x[b, k], W decoded from E2M1 codes with an E8M0
// scale per 32 columns (the unpack of the vLLM pull request 51583 digest,
// sections "功能与动机" and "实现拆解": the unpack feeds the MXFP4 MoE GEMM),
// accumulated in fp32.
//
// gfx950 design.
//   * Decode: v_cvt_scalef32_pk_bf16_fp4 turns one byte (two codes) into two
//     bf16 already multiplied by the block scale 2^(e-127); for 2 <= e <= 252
//     these are exactly the bf16 patterns of the lookup + exponent-add unpack
//     (zero codes give +/-0, which add nothing to a sum). v_dot2_f32_bf16
//     multiplies the pair by the matching pair of x and accumulates in fp32:
//     per byte of weights one conversion and one dot2.
//   * Batch 1 (the bandwidth-bound case): each lane owns fixed 32-column
//     chunks of K, so its slice of x sits in registers for the whole kernel
//     (staged once per workgroup through LDS). A group of G lanes covers one
//     row (G = 64 for K >= 2048, smaller for short rows so a wave works on
//     several rows at once); every weight byte is read once with a 16-byte
//     load, the next row is prefetched while the current one is reduced, and
//     the row total comes from a DPP / cross-row shuffle reduction.
//   * Other batches: one wave per row, lanes across K, x read through the
//     cache hierarchy per chunk.
#include "device.hpp"
#include "kernels.hpp"

namespace e2m1 {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;

// Dot product of one 32-column block (16 code bytes in w, scale s) with the 16
// x words (bf16 pairs) of the same columns. Two accumulators halve the
// dependency chain.
__device__ __forceinline__ float block_dot(const uint4 w, float s, const uint32_t* xw, float acc) {
    float a0 = 0.f, a1 = 0.f;
    a0 = dot2_bf16(fp4x2_to_bf16x2<0>(w.x, s), xw[0], a0);
    a1 = dot2_bf16(fp4x2_to_bf16x2<1>(w.x, s), xw[1], a1);
    a0 = dot2_bf16(fp4x2_to_bf16x2<2>(w.x, s), xw[2], a0);
    a1 = dot2_bf16(fp4x2_to_bf16x2<3>(w.x, s), xw[3], a1);
    a0 = dot2_bf16(fp4x2_to_bf16x2<0>(w.y, s), xw[4], a0);
    a1 = dot2_bf16(fp4x2_to_bf16x2<1>(w.y, s), xw[5], a1);
    a0 = dot2_bf16(fp4x2_to_bf16x2<2>(w.y, s), xw[6], a0);
    a1 = dot2_bf16(fp4x2_to_bf16x2<3>(w.y, s), xw[7], a1);
    a0 = dot2_bf16(fp4x2_to_bf16x2<0>(w.z, s), xw[8], a0);
    a1 = dot2_bf16(fp4x2_to_bf16x2<1>(w.z, s), xw[9], a1);
    a0 = dot2_bf16(fp4x2_to_bf16x2<2>(w.z, s), xw[10], a0);
    a1 = dot2_bf16(fp4x2_to_bf16x2<3>(w.z, s), xw[11], a1);
    a0 = dot2_bf16(fp4x2_to_bf16x2<0>(w.w, s), xw[12], a0);
    a1 = dot2_bf16(fp4x2_to_bf16x2<1>(w.w, s), xw[13], a1);
    a0 = dot2_bf16(fp4x2_to_bf16x2<2>(w.w, s), xw[14], a0);
    a1 = dot2_bf16(fp4x2_to_bf16x2<3>(w.w, s), xw[15], a1);
    return acc + (a0 + a1);
}

template <bool kBf16Out>
__device__ __forceinline__ void store_out(void* y, int64_t idx, float v) {
    if constexpr (kBf16Out)
        reinterpret_cast<uint16_t*>(y)[idx] = (uint16_t)f32_to_bf16_rne(v);
    else
        reinterpret_cast<float*>(y)[idx] = v;
}

// ------------------------------------------------------------- batch 1 ----

template <int G, int CPL>
__device__ __forceinline__ void load_row(const uint8_t* __restrict__ packed,
                                         const uint8_t* __restrict__ scales, int row, int n,
                                         int kc, int gl, uint4 (&w)[CPL], uint32_t (&e)[CPL]) {
#pragma unroll
    for (int ci = 0; ci < CPL; ++ci) {
        const int c = gl + G * ci;
        if (row < n && c < kc) {
            const int64_t blk = (int64_t)row * kc + c;
            w[ci] = load_nt16(reinterpret_cast<const uint4*>(packed) + blk);
            e[ci] = scales[blk];
        } else {
            w[ci] = make_uint4(0u, 0u, 0u, 0u);
            e[ci] = 0u;
        }
    }
}

template <int G, int CPL, bool kBf16Out>
__global__ __launch_bounds__(kThreads) void gemv_b1_kernel(const uint8_t* __restrict__ packed,
                                                           const uint8_t* __restrict__ scales,
                                                           const uint16_t* __restrict__ x,
                                                           void* __restrict__ y, int n, int kc) {
    extern __shared__ uint4 xs[];   // kc * 4 uint4 = all of x
    constexpr int kRowsPerWave = kWave / G;
    const int lane = threadIdx.x & (kWave - 1);
    const int gl = lane & (G - 1);
    const int grp = lane / G;
    const int wave = blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave);
    const int row_stride = gridDim.x * kWavesPerBlock * kRowsPerWave;
    int base = wave * kRowsPerWave;   // wave-uniform first row of this wave

    uint4 wcur[CPL];
    uint32_t ecur[CPL];
    load_row<G, CPL>(packed, scales, base + grp, n, kc, gl, wcur, ecur);

    for (int i = threadIdx.x; i < kc * 4; i += kThreads) xs[i] = reinterpret_cast<const uint4*>(x)[i];
    __syncthreads();
    uint32_t xr[CPL][16];
#pragma unroll
    for (int ci = 0; ci < CPL; ++ci) {
        const int c = gl + G * ci;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 v = (c < kc) ? xs[c * 4 + q] : make_uint4(0u, 0u, 0u, 0u);
            xr[ci][4 * q + 0] = v.x;
            xr[ci][4 * q + 1] = v.y;
            xr[ci][4 * q + 2] = v.z;
            xr[ci][4 * q + 3] = v.w;
        }
    }

    for (; base < n; base += row_stride) {
        uint4 wnxt[CPL];
        uint32_t enxt[CPL];
        load_row<G, CPL>(packed, scales, base + row_stride + grp, n, kc, gl, wnxt, enxt);
        float acc = 0.f;
#pragma unroll
        for (int ci = 0; ci < CPL; ++ci) acc = block_dot(wcur[ci], e8m0_as_f32(ecur[ci]), xr[ci], acc);
        acc = group_sum<G>(acc);
        const int row = base + grp;
        if (gl == 0 && row < n) store_out<kBf16Out>(y, row, acc);
#pragma unroll
        for (int ci = 0; ci < CPL; ++ci) {
            wcur[ci] = wnxt[ci];
            ecur[ci] = enxt[ci];
        }
    }
}

// --------------------------------------------------------- any batch ----

template <int B, bool kBf16Out>
__global__ __launch_bounds__(kThreads) void gemv_generic_kernel(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ scales,
    const uint16_t* __restrict__ x, void* __restrict__ y, int n, int kc) {
    const int lane = threadIdx.x & (kWave - 1);
    const int nwaves = gridDim.x * kWavesPerBlock;
    const uint4* xv = reinterpret_cast<const uint4*>(x);
    for (int row = blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; row < n; row += nwaves) {
        float acc[B];
#pragma unroll
        for (int b = 0; b < B; ++b) acc[b] = 0.f;
        for (int c = lane; c < kc; c += kWave) {
            const int64_t blk = (int64_t)row * kc + c;
            const uint4 w = load_nt16(reinterpret_cast<const uint4*>(packed) + blk);
            const float s = e8m0_as_f32(scales[blk]);
            uint32_t wd[16];
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                wd[4 * q + 0] = fp4x2_to_bf16x2<0>(ws[q], s);
                wd[4 * q + 1] = fp4x2_to_bf16x2<1>(ws[q], s);
                wd[4 * q + 2] = fp4x2_to_bf16x2<2>(ws[q], s);
                wd[4 * q + 3] = fp4x2_to_bf16x2<3>(ws[q], s);
            }
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const uint4* xp = xv + ((int64_t)b * kc + c) * 4;
                float a = acc[b];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint4 xq = xp[q];
                    a = dot2_bf16(wd[4 * q + 0], xq.x, a);
                    a = dot2_bf16(wd[4 * q + 1], xq.y, a);
                    a = dot2_bf16(wd[4 * q + 2], xq.z, a);
                    a = dot2_bf16(wd[4 * q + 3], xq.w, a);
                }
                acc[b] = a;
            }
        }
#pragma unroll
        for (int b = 0; b < B; ++b) acc[b] = group_sum<kWave>(acc[b]);
        if (lane == 0) {
#pragma unroll
            for (int b = 0; b < B; ++b) store_out<kBf16Out>(y, (int64_t)b * n + row, acc[b]);
        }
    }
}

// ------------------------------------------------------------- launch ----

template <typename Kernel>
int resident_blocks(Kernel kernel, size_t lds_bytes) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, lds_bytes) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    return per_cu * device_cu_count();
}

template <int G, int CPL, bool kBf16Out>
hipError_t run_b1(const uint8_t* packed, const uint8_t* scales, const uint16_t* x, void* y,
                  int n, int kc, hipStream_t stream) {
    auto kernel = gemv_b1_kernel<G, CPL, kBf16Out>;
    const size_t lds = (size_t)kc * 64;
    const int rows_per_block = kWavesPerBlock * (kWave / G);
    const int want = (n + rows_per_block - 1) / rows_per_block;
    // Residency with the most LDS this instantiation can ask for (kc <= G*CPL);
    // cached per instantiation, the same on every gfx950 device.
    static int cap = 0;
    if (cap == 0) cap = resident_blocks(kernel, (size_t)64 * G * CPL);
    const int grid = want < cap ? want : cap;
    kernel<<<grid, kThreads, lds, stream>>>(packed, scales, x, y, n, kc);
    return hipGetLastError();
}

template <bool kBf16Out>
hipError_t dispatch_b1(const uint8_t* packed, const uint8_t* scales, const uint16_t* x, void* y,
                       int n, int kc, hipStream_t stream) {
    if (kc <= 8) return run_b1<8, 1, kBf16Out>(packed, scales, x, y, n, kc, stream);
    if (kc <= 16) return run_b1<16, 1, kBf16Out>(packed, scales, x, y, n, kc, stream);
    if (kc <= 32) return run_b1<32, 1, kBf16Out>(packed, scales, x, y, n, kc, stream);
    switch ((kc + kWave - 1) / kWave) {
        case 1: return run_b1<64, 1, kBf16Out>(packed, scales, x, y, n, kc, stream);
        case 2: return run_b1<64, 2, kBf16Out>(packed, scales, x, y, n, kc, stream);
        case 3: return run_b1<64, 3, kBf16Out>(packed, scales, x, y, n, kc, stream);
        case 4: return run_b1<64, 4, kBf16Out>(packed, scales, x, y, n, kc, stream);
        case 5: return run_b1<64, 5, kBf16Out>(packed, scales, x, y, n, kc, stream);
        case 6: return run_b1<64, 6, kBf16Out>(packed, scales, x, y, n, kc, stream);
        case 7: return run_b1<64, 7, kBf16Out>(packed, scales, x, y, n, kc, stream);
        default: return run_b1<64, 8, kBf16Out>(packed, scales, x, y, n, kc, stream);
    }
}

template <int B, bool kBf16Out>
hipError_t run_generic(const uint8_t* packed, const uint8_t* scales, const uint16_t* x, void* y,
                       int n, int kc, hipStream_t stream) {
    auto kernel = gemv_generic_kernel<B, kBf16Out>;
    const int want = (n + kWavesPerBlock - 1) / kWavesPerBlock;
    static int cap = 0;
    if (cap == 0) cap = resident_blocks(kernel, 0);
    const int grid = want < cap ? want : cap;
    kernel<<<grid, kThreads, 0, stream>>>(packed, scales, x, y, n, kc);
    return hipGetLastError();
}

template <bool kBf16Out>
hipError_t dispatch_generic(int batch, const uint8_t* packed, const uint8_t* scales,
                            const uint16_t* x, void* y, int n, int kc, hipStream_t stream) {
#define E2M1_GEMV_CASE(B) \
    case B: return run_generic<B, kBf16Out>(packed, scales, x, y, n, kc, stream);
    switch (batch) {
        E2M1_GEMV_CASE(1) E2M1_GEMV_CASE(2) E2M1_GEMV_CASE(3) E2M1_GEMV_CASE(4)
        E2M1_GEMV_CASE(5) E2M1_GEMV_CASE(6) E2M1_GEMV_CASE(7) E2M1_GEMV_CASE(8)
        E2M1_GEMV_CASE(9) E2M1_GEMV_CASE(10) E2M1_GEMV_CASE(11) E2M1_GEMV_CASE(12)
        E2M1_GEMV_CASE(13) E2M1_GEMV_CASE(14) E2M1_GEMV_CASE(15) E2M1_GEMV_CASE(16)
        default: return hipErrorInvalidValue;
    }
#undef E2M1_GEMV_CASE
}

}  // namespace

// Largest K the batch-1 kernel keeps in registers (8 chunks of 32 per lane).
constexpr int64_t kB1MaxK = 64 * 8 * 32;

hipError_t launch_gemv(const uint8_t* packed, const uint8_t* scales, const uint16_t* x, void* y,
                       bool out_bf16, int batch, int64_t n, int64_t k, hipStream_t stream) {
    const int kc = (int)(k / 32);
    const int nn = (int)n;
    if (batch == 1 && k <= kB1MaxK)
        return out_bf16 ? dispatch_b1<true>(packed, scales, x, y, nn, kc, stream)
                        : dispatch_b1<false>(packed, scales, x, y, nn, kc, stream);
    return out_bf16 ? dispatch_generic<true>(batch, packed, scales, x, y, nn, kc, stream)
                    : dispatch_generic<false>(batch, packed, scales, x, y, nn, kc, stream);
}

}  // namespace e2m1
