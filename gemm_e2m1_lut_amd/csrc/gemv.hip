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
//     chunks of K, so its slice of x sits in registers for the whole kernel.
//     A group of G lanes covers one row (G = 64 for K >= 2048, smaller for
//     short rows so a wave works on several rows at once) and takes R
//     consecutive rows per pass, R sized so one resident generation of waves
//     covers the matrix. Every weight byte is read once with a 16-byte load,
//     all of a pass's loads are in flight before the first row is computed,
//     and the row total comes from a DPP-only reduction (row_bcast for the
//     cross-row steps), so the decode and dot products hide under the loads.
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

// Row total of groups of G lanes (G in {8, 16, 32, 64}) with DPP only: the
// total ends up in the last lane of each group (lane G-1 mod G).
template <int G>
__device__ __forceinline__ float group_total(float v) {
    v += dpp_f32<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp_f32<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp_f32<0x141>(v);   // row_half_mirror: every lane holds its 8-lane sum
    if constexpr (G >= 16) v += dpp_f32<0x140>(v);   // row_mirror: 16-lane sum
    if constexpr (G >= 32)   // row_bcast:15 into rows 1 and 3
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
    if constexpr (G >= 64)   // row_bcast:31 into rows 2 and 3
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));
    return v;
}

// Batch 1. A group of G lanes covers one row; lane gl owns the 32-column chunks
// gl, gl + G, ... (CPL of them) for every row it visits, so its slice of x is
// loaded once into registers. A group takes R consecutive rows per pass. All
// loads are unconditional (indices clamped into range, out-of-range lanes and
// rows masked at use): guarded loads with a zero in the other branch would
// make each load wait for the previous one. x is requested first, then every
// weight chunk and scale of the pass, so computing row 0 waits only for x and
// row 0 while the later rows are still in flight.
template <int G, int CPL, int R, bool kBf16Out>
__global__ __launch_bounds__(kThreads) void gemv_b1_kernel(const uint8_t* __restrict__ packed,
                                                           const uint8_t* __restrict__ scales,
                                                           const uint16_t* __restrict__ x,
                                                           void* __restrict__ y, int n, int kc) {
    constexpr int kGroupsPerWave = kWave / G;
    const int lane = threadIdx.x & (kWave - 1);
    const int gl = lane & (G - 1);
    const int grp = lane / G;
    const int wave = blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    const int units = gridDim.x * kWavesPerBlock * kGroupsPerWave;   // row groups in the grid
    const int unit = wave * kGroupsPerWave + grp;
    const uint4* xv = reinterpret_cast<const uint4*>(x);
    const uint4* pv = reinterpret_cast<const uint4*>(packed);

    uint32_t xr[CPL][16];
#pragma unroll
    for (int ci = 0; ci < CPL; ++ci) {
        const int c = min(gl + G * ci, kc - 1);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 v = xv[c * 4 + q];
            xr[ci][4 * q + 0] = v.x;
            xr[ci][4 * q + 1] = v.y;
            xr[ci][4 * q + 2] = v.z;
            xr[ci][4 * q + 3] = v.w;
        }
    }
    // wave-uniform pass count: passes while the wave's first group has rows
    for (int pass = 0; (pass * units + wave * kGroupsPerWave) * R < n; ++pass) {
        const int row0 = (pass * units + unit) * R;
        uint4 w[R][CPL];
        uint32_t e[R][CPL];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int ci = 0; ci < CPL; ++ci) {
                const int64_t blk = (int64_t)min(row0 + r, n - 1) * kc + min(gl + G * ci, kc - 1);
                w[r][ci] = load_nt16(pv + blk);
                e[r][ci] = scales[blk];
            }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float acc = 0.f;
#pragma unroll
            for (int ci = 0; ci < CPL; ++ci) {
                const uint4 wv = (gl + G * ci < kc) ? w[r][ci] : make_uint4(0u, 0u, 0u, 0u);
                acc = block_dot(wv, e8m0_scale(e[r][ci]), xr[ci], acc);
            }
            acc = group_total<G>(acc);
            if (gl == G - 1 && row0 + r < n) store_out<kBf16Out>(y, row0 + r, acc);
        }
    }
}

// Batch 1, long rows (K > 8192). Holding all of a row's x slice per wave
// would make every wave pull the whole of x through its compute unit, more
// bytes than the weights it streams. Here the WR waves of a workgroup split
// K: lane l of wave w owns the single chunk 64 w + l (16 x registers), the
// workgroup takes RB consecutive rows per pass, every wave reduces its part
// of each row with DPP, and the WR partial sums meet in LDS.
template <int WR, int RB, bool kBf16Out>
__global__ __launch_bounds__(kWave * WR) void gemv_b1_slab_kernel(const uint8_t* __restrict__ packed,
                                                                  const uint8_t* __restrict__ scales,
                                                                  const uint16_t* __restrict__ x,
                                                                  void* __restrict__ y, int n, int kc) {
    __shared__ float part[RB][WR];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wig = tid / kWave;
    const int c_raw = wig * kWave + lane;
    const bool cvalid = c_raw < kc;
    const int c = min(c_raw, kc - 1);
    const uint4* pv = reinterpret_cast<const uint4*>(packed);
    uint32_t xr[16];
    {
        const uint4* xv = reinterpret_cast<const uint4*>(x) + c * 4;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 v = xv[q];
            xr[4 * q + 0] = v.x;
            xr[4 * q + 1] = v.y;
            xr[4 * q + 2] = v.z;
            xr[4 * q + 3] = v.w;
        }
    }
    for (int rb = blockIdx.x * RB; rb < n; rb += gridDim.x * RB) {   // workgroup-uniform
        uint4 w[RB];
        uint32_t e[RB];
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            const int64_t blk = (int64_t)min(rb + i, n - 1) * kc + c;
            w[i] = load_nt16(pv + blk);
            e[i] = scales[blk];
        }
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            const uint4 wv = cvalid ? w[i] : make_uint4(0u, 0u, 0u, 0u);
            const float acc = group_total<kWave>(block_dot(wv, e8m0_scale(e[i]), xr, 0.f));
            if (lane == kWave - 1) part[i][wig] = acc;
        }
        __syncthreads();
        if (tid < RB && rb + tid < n) {
            float s = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < WR; ++w2) s += part[tid][w2];
            store_out<kBf16Out>(y, rb + tid, s);
        }
        __syncthreads();
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
            const float s = e8m0_scale(scales[blk]);
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
int resident_blocks(Kernel kernel, size_t lds_bytes, int threads = kThreads) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds_bytes) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    return per_cu * device_cu_count();
}

template <int G, int CPL, int R, bool kBf16Out>
hipError_t run_b1_r(const uint8_t* packed, const uint8_t* scales, const uint16_t* x, void* y, int n,
                    int kc, int cap, hipStream_t stream) {
    const int rows_per_block = kWavesPerBlock * (kWave / G) * R;
    const int want = (n + rows_per_block - 1) / rows_per_block;
    const int grid = want < cap ? want : cap;
    gemv_b1_kernel<G, CPL, R, kBf16Out><<<grid, kThreads, 0, stream>>>(packed, scales, x, y, n, kc);
    return hipGetLastError();
}

// Rows per group and pass: the fewest (1, 2 or 4) that let every row group of
// one resident wave generation finish the matrix in a single pass.
template <int G, int CPL, bool kBf16Out>
hipError_t run_b1(const uint8_t* packed, const uint8_t* scales, const uint16_t* x, void* y, int n,
                  int kc, hipStream_t stream) {
    static int cap1 = 0, cap2 = 0, cap4 = 0;   // resident blocks per R, same on every gfx950
    if (cap1 == 0) {
        cap1 = resident_blocks(gemv_b1_kernel<G, CPL, 1, kBf16Out>, 0);
        cap2 = resident_blocks(gemv_b1_kernel<G, CPL, 2, kBf16Out>, 0);
        cap4 = resident_blocks(gemv_b1_kernel<G, CPL, 4, kBf16Out>, 0);
    }
    const int groups_per_block = kWavesPerBlock * (kWave / G);
    if ((int64_t)cap1 * groups_per_block >= n)
        return run_b1_r<G, CPL, 1, kBf16Out>(packed, scales, x, y, n, kc, cap1, stream);
    if ((int64_t)cap2 * groups_per_block * 2 >= n || CPL > 4)
        return run_b1_r<G, CPL, 2, kBf16Out>(packed, scales, x, y, n, kc, cap2, stream);
    return run_b1_r<G, CPL, 4, kBf16Out>(packed, scales, x, y, n, kc, cap4, stream);
}

template <int WR, int RB, bool kBf16Out>
hipError_t run_slab_r(const uint8_t* packed, const uint8_t* scales, const uint16_t* x, void* y, int n,
                      int kc, int cap, hipStream_t stream) {
    const int want = (n + RB - 1) / RB;
    const int grid = want < cap ? want : cap;
    gemv_b1_slab_kernel<WR, RB, kBf16Out><<<grid, kWave * WR, 0, stream>>>(packed, scales, x, y, n, kc);
    return hipGetLastError();
}

// Rows per workgroup pass: the fewest (2, 4 or 8) that cover the matrix with
// one resident generation of workgroups.
template <int WR, bool kBf16Out>
hipError_t run_slab(const uint8_t* packed, const uint8_t* scales, const uint16_t* x, void* y, int n,
                    int kc, hipStream_t stream) {
    static int cap2 = 0, cap4 = 0, cap8 = 0;
    if (cap2 == 0) {
        cap2 = resident_blocks(gemv_b1_slab_kernel<WR, 2, kBf16Out>, 0, kWave * WR);
        cap4 = resident_blocks(gemv_b1_slab_kernel<WR, 4, kBf16Out>, 0, kWave * WR);
        cap8 = resident_blocks(gemv_b1_slab_kernel<WR, 8, kBf16Out>, 0, kWave * WR);
    }
    if ((int64_t)cap2 * 2 >= n) return run_slab_r<WR, 2, kBf16Out>(packed, scales, x, y, n, kc, cap2, stream);
    if ((int64_t)cap4 * 4 >= n) return run_slab_r<WR, 4, kBf16Out>(packed, scales, x, y, n, kc, cap4, stream);
    return run_slab_r<WR, 8, kBf16Out>(packed, scales, x, y, n, kc, cap8, stream);
}

template <bool kBf16Out>
hipError_t dispatch_b1(const uint8_t* packed, const uint8_t* scales, const uint16_t* x, void* y,
                       int n, int kc, hipStream_t stream) {
    if (kc > 4 * kWave) {
        switch ((kc + kWave - 1) / kWave) {
            case 5: return run_slab<5, kBf16Out>(packed, scales, x, y, n, kc, stream);
            case 6: return run_slab<6, kBf16Out>(packed, scales, x, y, n, kc, stream);
            case 7: return run_slab<7, kBf16Out>(packed, scales, x, y, n, kc, stream);
            case 8: return run_slab<8, kBf16Out>(packed, scales, x, y, n, kc, stream);
            case 9: return run_slab<9, kBf16Out>(packed, scales, x, y, n, kc, stream);
            case 10: return run_slab<10, kBf16Out>(packed, scales, x, y, n, kc, stream);
            case 11: return run_slab<11, kBf16Out>(packed, scales, x, y, n, kc, stream);
            case 12: return run_slab<12, kBf16Out>(packed, scales, x, y, n, kc, stream);
            case 13: return run_slab<13, kBf16Out>(packed, scales, x, y, n, kc, stream);
            case 14: return run_slab<14, kBf16Out>(packed, scales, x, y, n, kc, stream);
            case 15: return run_slab<15, kBf16Out>(packed, scales, x, y, n, kc, stream);
            default: return run_slab<16, kBf16Out>(packed, scales, x, y, n, kc, stream);
        }
    }
    if (kc <= 8) return run_b1<8, 1, kBf16Out>(packed, scales, x, y, n, kc, stream);
    if (kc <= 16) return run_b1<16, 1, kBf16Out>(packed, scales, x, y, n, kc, stream);
    if (kc <= 32) return run_b1<32, 1, kBf16Out>(packed, scales, x, y, n, kc, stream);
    switch ((kc + kWave - 1) / kWave) {
        case 1: return run_b1<64, 1, kBf16Out>(packed, scales, x, y, n, kc, stream);
        case 2: return run_b1<64, 2, kBf16Out>(packed, scales, x, y, n, kc, stream);
        case 3: return run_b1<64, 3, kBf16Out>(packed, scales, x, y, n, kc, stream);
        default: return run_b1<64, 4, kBf16Out>(packed, scales, x, y, n, kc, stream);
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

// Largest K of the batch-1 kernels: 16 waves of 64 lanes, one 32-column chunk
// per lane (the register-resident kernel stops at 4 chunks per lane, K = 8192).
constexpr int64_t kB1MaxK = 16 * 64 * 32;

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
