// gemm.hip -- MXFP4 weight GEMM for many activation rows (dequant_gemm): the
// prefill counterpart of dequant_gemv.
//
// Semantics: y[m][n] = sum_k dec(W)[n][k] x[m][k] with fp32 accumulation, W
// MXFP4 (E2M1 codes + one E8M0 scale per 32 columns, the unpack of the vLLM
// pull request 51583 digest, section "功能与动机"), x bf16. The digest's
// comment section describes the CPU GEMM decoding each weight block into a
// bf16 tile before the multiply ("decode to tile"); here the decode feeds the
// matrix cores directly.
//
// gfx950 design. With hundreds of activation rows the product is bound by
// the matrix cores (2 m flops per 0.53 bytes of weights), so the kernel is a
// tiled bf16 MFMA GEMM whose weight operand is decoded on the way in:
//   * A workgroup of four waves owns a tile of 128 weight rows x 128
//     activation rows and walks K in steps of 64 columns. Each step, its
//     threads copy the step's x tile (128 x 64 bf16) and the raw code lines
//     (128 rows x 32 bytes) and scale bytes of W into LDS with coalesced
//     16-byte loads, double-buffered: the loads of step s + 1 are issued
//     before the MFMAs of step s and written to the other buffer after them,
//     with one barrier per step.
//   * Waves are laid out 2 x 2 over the tile; each owns 64 weight rows x 64
//     activation rows as 4 x 4 tiles of v_mfma_f32_16x16x32_bf16. Lane
//     l = 16 g + r takes 8 codes (4 bytes) of weight row r per 32 columns and
//     decodes them with four v_cvt_scalef32_pk_bf16_fp4 (two codes each, table
//     lookup and E8M0 scale in one instruction); every decoded A operand
//     serves the wave's four activation tiles, so decoding costs one
//     instruction per MFMA.
//     B operands are 16-byte LDS reads of x at the same columns.
//   * D element (weight row 4 g + j, activation row c) sits in lane 16 g + c,
//     so each lane stores four consecutive outputs of one row of y.
// Rows past N or M are loaded clamped and not stored; a 32-column half step
// past K is decoded as zero weights.
#include "device.hpp"
#include "kernels.hpp"

namespace e2m1 {
namespace {

constexpr int kThreads = 256;
constexpr int kTileN = 128;                  // weight rows per workgroup
constexpr int kTileM = 128;                  // activation rows per workgroup
constexpr int kStepK = 64;                   // columns per step
constexpr int kXPitch = kStepK + 8;          // bf16 per staged x row (16-byte pad spreads the banks)
constexpr int kWPitch = 32 + 4;              // bytes per staged code row
constexpr int kXElems = kTileM * kXPitch;
constexpr int kWBytes = kTileN * kWPitch;

struct GemmBuf {
    uint16_t x[kXElems];
    uint8_t w[kWBytes];
    uint8_t s[kTileN * 2];
};

template <bool kBf16Out>
__device__ __forceinline__ void store4(void* y, int64_t idx, const f32x4& v, bool full, int count) {
    if constexpr (kBf16Out) {
        uint16_t* p = reinterpret_cast<uint16_t*>(y) + idx;
        if (full && (idx & 3) == 0) {
            *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        } else {
            for (int j = 0; j < count; ++j) p[j] = (uint16_t)f32_to_bf16_rne(v[j]);
        }
    } else {
        float* p = reinterpret_cast<float*>(y) + idx;
        if (full && (idx & 3) == 0) {
            *reinterpret_cast<f32x4*>(p) = v;
        } else {
            for (int j = 0; j < count; ++j) p[j] = v[j];
        }
    }
}

template <bool kBf16Out>
__global__ __launch_bounds__(kThreads) void gemm_kernel(const uint8_t* __restrict__ packed,
                                                        const uint8_t* __restrict__ scales,
                                                        const uint16_t* __restrict__ x, void* __restrict__ y,
                                                        int m_rows, int n, int kc) {
    __shared__ __attribute__((aligned(16))) GemmBuf buf[2];
    const int t = threadIdx.x;
    const int lane = t & (kWave - 1);
    const int wave = t / kWave;
    const int g = lane >> 4, r = lane & 15;
    const int wn = (wave & 1) * 64, wm = (wave >> 1) * 64;   // the wave's quarter of the tile
    const int K = kc * 32;
    const int nsteps = (kc + 1) / 2;
    const int ntn = (n + kTileN - 1) / kTileN;
    const int n0 = (blockIdx.x % ntn) * kTileN;
    const int m0 = (blockIdx.x / ntn) * kTileM;

    // this thread's share of a step's copies: x chunks t + 256 i (row id / 8, 8 columns each),
    // code line t (row t / 2, 32-column block t % 2), scale bytes of row t (t < 128)
    const uint16_t* xsrc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) xsrc[i] = x + (size_t)min(m0 + ((t + kThreads * i) >> 3), m_rows - 1) * K;
    const int xcol = 8 * (t & 7);   // the same for the four chunks (kThreads is a multiple of 8)
    const uint8_t* wsrc = packed + (size_t)min(n0 + (t >> 1), n - 1) * (K / 2);
    const uint8_t* ssrc = scales + (size_t)min(n0 + (t & 127), n - 1) * kc;

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint4 xr[4], wr;
    uint32_t sr;
// Step `st`'s copies into registers. Columns past K (the second half of a last
// half step) read the row's last 8 columns: finite values that meet zero weights.
#define E2M1_GEMM_ISSUE(st)                                                                             \
    {                                                                                                   \
        const int c0 = (st) * kStepK;                                                                   \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) xr[i] =                                          \
            *reinterpret_cast<const uint4*>(xsrc[i] + min(c0 + xcol, K - 8));                          \
        wr = *reinterpret_cast<const uint4*>(wsrc + (size_t)min(2 * (st) + (t & 1), kc - 1) * 16);      \
        sr = (uint32_t)ssrc[min(2 * (st), kc - 1)] | ((uint32_t)ssrc[min(2 * (st) + 1, kc - 1)] << 8);  \
    }
// The registers of step `st` into buffer `bb`; a block past K is staged as zero codes.
#define E2M1_GEMM_STAGE(bb, st)                                                                          \
    {                                                                                                   \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                                 \
            const int id = t + kThreads * i;                                                            \
            *reinterpret_cast<uint4*>((bb).x + (id >> 3) * kXPitch + 8 * (id & 7)) = xr[i];             \
        }                                                                                               \
        const uint32_t keep = 2 * (st) + (t & 1) < kc ? 0xFFFFFFFFu : 0u;                               \
        uint32_t* wd = reinterpret_cast<uint32_t*>((bb).w + (t >> 1) * kWPitch + 16 * (t & 1));          \
        wd[0] = wr.x & keep;                                                                            \
        wd[1] = wr.y & keep;                                                                            \
        wd[2] = wr.z & keep;                                                                            \
        wd[3] = wr.w & keep;                                                                            \
        if (t < kTileN) *reinterpret_cast<uint16_t*>((bb).s + 2 * t) = (uint16_t)sr;                    \
    }

    E2M1_GEMM_ISSUE(0)
    E2M1_GEMM_STAGE(buf[0], 0)
    __syncthreads();
    for (int step = 0; step < nsteps; ++step) {
        const GemmBuf& b = buf[step & 1];
        // the next step's copies (the last step repeats its own: staged into the idle buffer, never read)
        const int nxt = min(step + 1, nsteps - 1);
        E2M1_GEMM_ISSUE(nxt)
        asm volatile("" ::: "memory");        // the loads stay here, ahead of the step's MFMAs
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int h = 0; h < 2; ++h) {   // 32-column half steps
            bf16x8 a[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = wn + 16 * i + r;
                const uint32_t codes = *reinterpret_cast<const uint32_t*>(b.w + row * kWPitch + 16 * h + 4 * g);
                const float sc = e8m0_scale(b.s[2 * row + h]);
                const u32x4 u = {fp4x2_to_bf16x2<0>(codes, sc), fp4x2_to_bf16x2<1>(codes, sc),
                                 fp4x2_to_bf16x2<2>(codes, sc), fp4x2_to_bf16x2<3>(codes, sc)};
                a[i] = __builtin_bit_cast(bf16x8, u);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bf16x8 bx = *reinterpret_cast<const bf16x8*>(b.x + (wm + 16 * j + r) * kXPitch + 32 * h + 8 * g);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bx, acc[i][j], 0, 0, 0);
            }
        }
        E2M1_GEMM_STAGE(buf[(step + 1) & 1], nxt)
        __syncthreads();
    }
#undef E2M1_GEMM_ISSUE
#undef E2M1_GEMM_STAGE

    // lane (g, c) holds rows n0 + wn + 16 i + 4 g .. + 3 of activation row m0 + wm + 16 j + c
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int m = m0 + wm + 16 * j + r;
        if (m >= m_rows) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int nn = n0 + wn + 16 * i + 4 * g;
            if (nn >= n) continue;
            const int count = min(4, n - nn);
            store4<kBf16Out>(y, (int64_t)m * n + nn, acc[i][j], count == 4, count);
        }
    }
}

}  // namespace

hipError_t launch_gemm(const uint8_t* packed, const uint8_t* scales, const uint16_t* x, void* y, bool out_bf16,
                       int64_t m, int64_t n, int64_t k, hipStream_t stream) {
    const int ntn = (int)((n + kTileN - 1) / kTileN);
    const int ntm = (int)((m + kTileM - 1) / kTileM);
    const dim3 grid((unsigned)(ntn * ntm));
    if (out_bf16)
        gemm_kernel<true><<<grid, kThreads, 0, stream>>>(packed, scales, x, y, (int)m, (int)n, (int)(k / 32));
    else
        gemm_kernel<false><<<grid, kThreads, 0, stream>>>(packed, scales, x, y, (int)m, (int)n, (int)(k / 32));
    return hipGetLastError();
}

}  // namespace e2m1
