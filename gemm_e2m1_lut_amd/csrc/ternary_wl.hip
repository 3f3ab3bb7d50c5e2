// ternary_wl.hip -- widely-linear complex ternary GEMV (ternary_wl_gemv).
//
// Method: FairyFuse blog post, section "复杂值广泛线性层的融合核调度": a
// complex layer y = U x + W conj(x) whose matrices have ternary real and
// imaginary parts, evaluated as eight coupled real ternary GEMVs in one pass
// over the weights: each decoded weight serves both the real and the
// imaginary part of x (mask reuse), x is prepared once for all eight (input
// reuse), the conjugate enters as a sign and never as a second copy of x, and
// the eight partial sums stay in registers until the final reduction. Each of
// U_re, U_im, W_re, W_im is packed like the real ternary GEMV (section
// "三元 GEMV 的乘法消除原理": 16 weights per word, bit 2j+1 = +1, bit 2j = -1)
// with its own per-row scale, applied once after the row sum.
//
// gfx950 design. The eight sub-GEMVs are a contraction of four ternary
// matrices against a few columns derived from x, so the fast kernel runs them
// on the matrix cores with exact integer arithmetic:
//   * A operand: ternary weights as int8 -1 / 0 / +1. One mask of a shifted
//     word gives the fields j, j + 4, j + 8, j + 12 as v_perm_b32 selectors
//     into a 4-byte pool, so one perm decodes four weights (11 VALU
//     operations per 16-weight word).
//   * B operand: x_re and x_im in fixed point with one exponent S per part
//     and 256-column slice (from the slice's largest |x|): x 2^S = H +
//     L 2^-30, H the integer part and L the rounded fraction in units of
//     2^-30, each written as four signed base-256 digits (one add and one xor
//     of 0x00808080 turn an integer into its digit bytes). The sixteen digit
//     columns (H and L of x_re, then of x_im) fill the B operand.
//   * v_mfma_i32_16x16x64_i8 sums ternary times digit exactly in int32; per
//     slice digit column i of H is scaled by 2^(8 i - S) into fp32, of L by
//     2^(8 i - S - 30).
// So every row sum is exact for x on its slice's grid of 2^(-S-30): every
// element of at least 2^-36 times its slice's largest |x| is used exactly,
// any other to within 2^-60 times that largest, and the only other roundings
// are a few fp32 additions per row.

// Work split: a workgroup owns a tile of 16 rows (one workgroup per tile); its waves take 256-column
// slices (slice s of wave w = w, w + waves, ...). Lane l = 16 g + r loads the
// 16-byte chunk 4 s + g of row r of each matrix (four words, 64 columns) and
// decodes word q as the A operand of one MFMA; in that operand byte b of
// dword j is the weight of column 16 q + j + 4 b of the chunk, and the B
// operand of lane 16 g + c holds digit column c for the same columns in the
// same order, so the sum over k is complete. Each wave prepares the digits of
// its own slice (lane l: columns 16 q + j + 4 b of chunk l >> 4, word
// l >> 2 & 3, dword j = l & 3, b = 0..3, for both parts) in its own LDS area
// and reads them back as B operands, with no workgroup barrier. D element
// (row 4 g + j, column c) sits in component j of lane 16 g + c: the eight
// digit columns of each part are added by DPP within each 16-lane row, the
// waves through LDS, and one thread per row and component applies the four
// scales and the signs of the complex product. Inputs the fast kernel cannot take
// (K % 64 != 0, unaligned matrices) use a one-wave-per-row kernel that adds,
// subtracts or skips each x directly in fp32.
#include "device.hpp"
#include "kernels.hpp"
#include "ternary_int8.hpp"

namespace e2m1 {
namespace {

constexpr int kMaxWaves = 16;
constexpr int kSliceChunks = 4;                          // 64-column chunks per wave slice
constexpr int kVariants = 16;                            // H then L digits of x_re, then of x_im
constexpr int kRowPitch = 20;                            // dwords per row in LDS (spreads the banks)
// dwords per chunk: 16 more than its rows, so the four chunks' rows start 16 banks apart and the
// digit writes of a wave (one dword per lane, the four chunks side by side) meet no bank twice
constexpr int kChunkPitch = kVariants * kRowPitch + 16;
constexpr int kWaveDwords = kSliceChunks * kChunkPitch;
constexpr int kPartFloats = 4 * 2 * 16;                  // (matrix, part, row) partial sums

struct WlMats {
    const uint32_t* m[4];   // U_re, U_im, W_re, W_im
};

size_t wl_lds_bytes(int waves) {
    return 4u * ((size_t)waves * kWaveDwords + (size_t)waves * kPartFloats + kPartFloats);
}

// Fast kernel: K % 64 == 0, matrices 16-byte aligned.
__global__ __launch_bounds__(kWave * kMaxWaves) void ternary_wl_kernel(WlMats mats, const float* scale,
                                                                       const float* x_re, const float* x_im,
                                                                       float* y_re, float* y_im, int n, int kq) {
    extern __shared__ __attribute__((aligned(16))) uint32_t wl_smem[];
    const int nwaves = blockDim.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    uint32_t* tab = wl_smem + wave * kWaveDwords;
    float* part = reinterpret_cast<float*>(wl_smem + nwaves * kWaveDwords);
    float* tot = part + nwaves * kPartFloats;
    const int g = lane >> 4, r = lane & 15, c = lane & 15;
    const int K = 64 * kq;
    const int nslices = (kq + kSliceChunks - 1) / kSliceChunks;
    // digit preparation: lane -> chunk pg, word pq, dword pj; columns 64 pg + 16 pq + pj + 4 b
    const int pg = lane >> 4, pq = (lane >> 2) & 3, pj = lane & 3;
    uint32_t* prep_row = tab + pg * kChunkPitch + 4 * pq + pj;
    const i32x4* b_row = reinterpret_cast<const i32x4*>(tab + g * kChunkPitch + c * kRowPitch);
    // digit column c: part c >> 3 (x_re, x_im), fraction digits for c & 4, digit c & 3
    const bool c_im = c & 8;
    const int c_shift = 8 * (c & 3) - ((c & 4) ? 30 : 0);

    const int tile = blockIdx.x;   // one tile of 16 rows per workgroup
    const int row = min(tile * 16 + r, n - 1);
    float sc[4] = {0.f, 0.f, 0.f, 0.f};
    if (wave == 0) {
#pragma unroll
        for (int m = 0; m < 4; ++m) sc[m] = scale[(int64_t)m * n + row];
    }
    float f[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) f[m][j] = 0.f;

    for (int sl = wave; sl < nslices; sl += nwaves) {   // wave-uniform
        float xr[4], xi[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int col = min(256 * sl + 64 * pg + 16 * pq + pj + 4 * b, K - 1);
            xr[b] = x_re[col];
            xi[b] = x_im[col];
        }
        issue_fence();
        const int chunk = sl * kSliceChunks + g;
        const int cc = min(chunk, kq - 1);
        const uint32_t mask = chunk < kq ? 0xFFFFFFFFu : 0u;
        uint4 w[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) w[m] = load_nt16(mats.m[m] + ((int64_t)row * kq + cc) * 4);
        issue_fence();
        // digits of this slice's x into the wave's LDS area
        const int Sr = slice_exponent(wave_max(fmaxf(fmaxf(fabsf(xr[0]), fabsf(xr[1])),
                                                     fmaxf(fabsf(xr[2]), fabsf(xr[3])))));
        const int Si = slice_exponent(wave_max(fmaxf(fmaxf(fabsf(xi[0]), fabsf(xi[1])),
                                                     fmaxf(fabsf(xi[2]), fabsf(xi[3])))));
        uint32_t hr[4], lr[4], hi_[4], li[4], t[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            digits8(xr[b], Sr, hr[b], lr[b]);
            digits8(xi[b], Si, hi_[b], li[b]);
        }
        transpose4(hr, t);
#pragma unroll
        for (int i = 0; i < 4; ++i) prep_row[i * kRowPitch] = t[i];
        transpose4(lr, t);
#pragma unroll
        for (int i = 0; i < 4; ++i) prep_row[(4 + i) * kRowPitch] = t[i];
        transpose4(hi_, t);
#pragma unroll
        for (int i = 0; i < 4; ++i) prep_row[(8 + i) * kRowPitch] = t[i];
        transpose4(li, t);
#pragma unroll
        for (int i = 0; i < 4; ++i) prep_row[(12 + i) * kRowPitch] = t[i];
        __builtin_amdgcn_wave_barrier();   // LDS accesses of one wave complete in order
        i32x4 bq[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) bq[q] = b_row[q];
        i32x4 acc[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[m] = i32x4{0, 0, 0, 0};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const uint32_t ws[4] = {w[m].x, w[m].y, w[m].z, w[m].w};
                acc[m] = __builtin_amdgcn_mfma_i32_16x16x64_i8(decode_word(ws[q] & mask), bq[q], acc[m], 0, 0, 0);
            }
        }
        // digit column c is worth 2^(c_shift - S) of its part; |acc| <= 2^15, exact in fp32
        const int e = c_shift - (c_im ? Si : Sr);
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j) f[m][j] += ldexpf((float)acc[m][j], e);
        __builtin_amdgcn_wave_barrier();   // the B reads are done before the next slice's digits
    }

    // digits of x_re (columns 0..7) and of x_im (8..15): the sums land in lanes c = 7 and c = 15
    float s[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float v = f[m][j];
            v += dpp_f32<0x111>(v);   // row_shr:1
            v += dpp_f32<0x112>(v);   // row_shr:2
            v += dpp_f32<0x114>(v);   // row_shr:4
            s[m][j] = v;
        }
    if (c == 7 || c == 15) {
        float* dst = part + wave * kPartFloats + (c == 15 ? 16 : 0) + 4 * g;
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j) dst[32 * m + j] = s[m][j];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kPartFloats; i += blockDim.x) {   // one-wave workgroups take two rounds
        float sum = 0.f;
        for (int wv = 0; wv < nwaves; ++wv) sum += part[wv * kPartFloats + i];
        tot[i] = sum;
    }
    __syncthreads();
    const int t = threadIdx.x;
    if (t < 32) {
        const int rr = t & 15, orow = tile * 16 + rr;
        // tot[(2 m + p) 16 + row]: ternary row sum of matrix m against x_re (p = 0) or x_im (p = 1)
        const float ur_re = tot[0 * 16 + rr], ur_im = tot[1 * 16 + rr];
        const float ui_re = tot[2 * 16 + rr], ui_im = tot[3 * 16 + rr];
        const float wr_re = tot[4 * 16 + rr], wr_im = tot[5 * 16 + rr];
        const float wi_re = tot[6 * 16 + rr], wi_im = tot[7 * 16 + rr];
        float y;
        if (t < 16)   // Re: U_re x_re - U_im x_im + W_re x_re + W_im x_im
            y = (sc[0] * ur_re - sc[1] * ui_im) + (sc[2] * wr_re + sc[3] * wi_im);
        else          // Im: U_re x_im + U_im x_re - W_re x_im + W_im x_re
            y = (sc[0] * ur_im + sc[1] * ui_re) + (sc[3] * wi_re - sc[2] * wr_im);
        if (orow < n) (t < 16 ? y_re : y_im)[orow] = y;
    }
}

// Any K % 16 == 0: one wave per row, lanes across words, x from memory; the
// eight sub-GEMV sums are kept apart and combined once per row.
__global__ __launch_bounds__(256) void ternary_wl_generic_kernel(WlMats mats, const float* __restrict__ scale,
                                                                 const float* __restrict__ x_re,
                                                                 const float* __restrict__ x_im,
                                                                 float* __restrict__ y_re,
                                                                 float* __restrict__ y_im, int n, int kw) {
    const int lane = threadIdx.x & (kWave - 1);
    const int nw = gridDim.x * (blockDim.x / kWave);
    for (int row = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave; row < n; row += nw) {
        float sre[4] = {0.f, 0.f, 0.f, 0.f}, sim[4] = {0.f, 0.f, 0.f, 0.f};
        for (int wi = lane; wi < kw; wi += kWave) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const uint32_t word = mats.m[m][(int64_t)row * kw + wi];
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const uint32_t f = (word >> (2 * j)) & 3u;
                    const float xr = x_re[16 * wi + j], xi = x_im[16 * wi + j];
                    if (f == 2u) {
                        sre[m] += xr;
                        sim[m] += xi;
                    } else if (f == 1u) {
                        sre[m] -= xr;
                        sim[m] -= xi;
                    }
                }
            }
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            sre[m] = group_sum<kWave>(sre[m]);
            sim[m] = group_sum<kWave>(sim[m]);
        }
        if (lane == 0) {
            float s[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) s[m] = scale[(int64_t)m * n + row];
            y_re[row] = (s[0] * sre[0] - s[1] * sim[1]) + (s[2] * sre[2] + s[3] * sim[3]);
            y_im[row] = (s[0] * sim[0] + s[1] * sre[1]) + (s[3] * sre[3] - s[2] * sim[2]);
        }
    }
}

}  // namespace

hipError_t launch_ternary_wl(const uint32_t* const mats[4], const float* scale, const float* x_re,
                             const float* x_im, float* y_re, float* y_im, int64_t n, int64_t k,
                             hipStream_t stream) {
    const WlMats wm{{mats[0], mats[1], mats[2], mats[3]}};
    const int nn = (int)n;
    bool aligned = k % 64 == 0;
    for (int m = 0; m < 4; ++m) aligned = aligned && (reinterpret_cast<uintptr_t>(mats[m]) & 15u) == 0;
    if (aligned) {
        const int kq = (int)(k / 64);
        const int waves = min(kMaxWaves, (kq + kSliceChunks - 1) / kSliceChunks);
        const size_t lds = wl_lds_bytes(waves);
        const int ntiles = (nn + 15) / 16;   // one workgroup per tile: the hardware streams through them
        ternary_wl_kernel<<<ntiles, kWave * waves, lds, stream>>>(wm, scale, x_re, x_im, y_re, y_im, nn, kq);
        return hipGetLastError();
    }
    const int want = (nn + 3) / 4;
    const int grid = min(want, 8 * device_cu_count());
    ternary_wl_generic_kernel<<<grid, 256, 0, stream>>>(wm, scale, x_re, x_im, y_re, y_im, nn, (int)(k / 16));
    return hipGetLastError();
}

}  // namespace e2m1
