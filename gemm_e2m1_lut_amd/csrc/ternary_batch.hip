// ternary_batch.hip -- small-batch ternary GEMM (ternary_gemm).
//
// Method: the ternary GEMV of the FairyFuse blog post (section
// "三元 GEMV 的乘法消除原理": 16 weights per word, bit 2j+1 = +1, bit 2j = -1,
// the per-row scale applied once after the row sum) for a few activation rows
// at once; section "总结与启示" names this batched fusion for speculative
// decoding as the next step. Every weight is decoded once for all rows.
//
// gfx950 design: the int8 matrix-core formulation of ternary_int8.hpp. Each
// group of four activation rows fills the sixteen B columns of one
// v_mfma_i32_16x16x64_i8 (row 4 gi + b of group gi in columns 4 b .. 4 b + 3,
// one per base-256 digit), so a decoded A operand serves ceil(batch / 4)
// MFMAs; the int32 sums are exact and each digit column is scaled into fp32
// per 256-column slice. A workgroup owns a tile of 16 output rows and its
// waves take 256-column slices; lane l = 16 g + r loads the 16-byte chunk
// 4 s + g of row r (four words) and decodes word q as the A operand of one
// MFMA per group. Each wave writes the digits of its own slice into its own
// LDS area (lane l: columns 16 q + j + 4 b of chunk l >> 4, word l >> 2 & 3,
// dword j = l & 3, b = 0..3, of every row of the group) and reads them back as
// B operands, with no workgroup barrier. D element (output row 4 g + j,
// column c) is component j of lane 16 g + c; the four digit columns of each
// activation row are added by DPP, the waves through LDS, and the row scale
// multiplies the total once. Inputs the fast kernel cannot take (K % 64 != 0,
// unaligned weights) run the ternary GEMV once per activation row.
#include "device.hpp"
#include "kernels.hpp"
#include "ternary_int8.hpp"

namespace e2m1 {
namespace {

constexpr int kMaxWaves = 16;
constexpr int kSliceChunks = 4;                               // 64-column chunks per wave slice
constexpr int kColumns = 16;                                  // B columns: 4 rows x 4 digits
constexpr int kRowPitch = 20;                                 // dwords per (chunk, column) row in LDS
constexpr int kWaveDwords = kSliceChunks * kColumns * kRowPitch;

size_t gemm_lds_bytes(int waves, int groups) {
    return 4u * ((size_t)waves * kWaveDwords + (size_t)waves * groups * 64 + (size_t)groups * 64);
}

template <int NG>
__global__ __launch_bounds__(kWave * kMaxWaves) void ternary_gemm_kernel(const uint32_t* packed,
                                                                         const float* scale, const float* x,
                                                                         float* y, int batch, int n, int kq) {
    extern __shared__ __attribute__((aligned(16))) uint32_t tg_smem[];
    const int nwaves = blockDim.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    uint32_t* tab = tg_smem + wave * kWaveDwords;
    float* part = reinterpret_cast<float*>(tg_smem + nwaves * kWaveDwords);   // [waves][NG * 4 rows][16]
    float* tot = part + nwaves * NG * 64;                                     // [NG * 4 rows][16]
    const int g = lane >> 4, r = lane & 15, c = lane & 15;
    const int K = 64 * kq;
    const int nslices = (kq + kSliceChunks - 1) / kSliceChunks;
    const int ntiles = (n + 15) / 16;
    // digit preparation: lane -> chunk pg, word pq, dword pj; columns 64 pg + 16 pq + pj + 4 b
    const int pg = lane >> 4, pq = (lane >> 2) & 3, pj = lane & 3;
    uint32_t* prep_row = tab + pg * kColumns * kRowPitch + 4 * pq + pj;
    const i32x4* b_row = reinterpret_cast<const i32x4*>(tab + (g * kColumns + c) * kRowPitch);

    for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {   // workgroup-uniform
        const int row = min(tile * 16 + r, n - 1);
        float f[NG][4];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi)
#pragma unroll
            for (int j = 0; j < 4; ++j) f[gi][j] = 0.f;

        for (int sl = wave; sl < nslices; sl += nwaves) {   // wave-uniform
            const int col0 = 256 * sl + 64 * pg + 16 * pq + pj;
            float xv[4][4];   // [row of the group][b]
#pragma unroll
            for (int bl = 0; bl < 4; ++bl) {
                if (bl > 0 && bl >= batch) break;   // uniform: rows past the batch are not prepared
                const float* xr = x + (int64_t)bl * K;
#pragma unroll
                for (int b = 0; b < 4; ++b) xv[bl][b] = xr[min(col0 + 4 * b, K - 1)];
            }
            issue_fence();
            const int chunk = sl * kSliceChunks + g;
            const int cc = min(chunk, kq - 1);
            const uint32_t mask = chunk < kq ? 0xFFFFFFFFu : 0u;
            const uint4 w = load_nt16(packed + ((int64_t)row * kq + cc) * 4);
            issue_fence();
            i32x4 a[4];
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                const int rows = min(4, batch - 4 * gi);   // rows of this group (uniform, >= 1)
                if (gi > 0) {   // next group's activations
#pragma unroll
                    for (int bl = 0; bl < 4; ++bl) {
                        if (bl >= rows) break;
                        const float* xr = x + (int64_t)(4 * gi + bl) * K;
#pragma unroll
                        for (int b = 0; b < 4; ++b) xv[bl][b] = xr[min(col0 + 4 * b, K - 1)];
                    }
                }
                // digit columns of rows past the batch keep whatever integers LDS holds: their
                // D columns are never read
                int S[4] = {30, 30, 30, 30};
#pragma unroll
                for (int bl = 0; bl < 4; ++bl) {
                    if (bl >= rows) break;
                    S[bl] = slice_exponent(wave_max(fmaxf(fmaxf(fabsf(xv[bl][0]), fabsf(xv[bl][1])),
                                                          fmaxf(fabsf(xv[bl][2]), fabsf(xv[bl][3])))));
                    uint32_t d[4], t[4];
#pragma unroll
                    for (int b = 0; b < 4; ++b) d[b] = digits(xv[bl][b], S[bl]);
                    transpose4(d, t);
#pragma unroll
                    for (int i = 0; i < 4; ++i) prep_row[(4 * bl + i) * kRowPitch] = t[i];
                }
                if (gi == 0) {   // the weights are decoded once, after the first digits
                    const uint32_t ws[4] = {w.x & mask, w.y & mask, w.z & mask, w.w & mask};
#pragma unroll
                    for (int q = 0; q < 4; ++q) a[q] = decode_word(ws[q]);
                }
                __builtin_amdgcn_wave_barrier();   // LDS accesses of one wave complete in order
                i32x4 acc = {0, 0, 0, 0};
#pragma unroll
                for (int q = 0; q < 4; ++q) acc = mfma_i8(a[q], b_row[q], acc);
                // column c: digit c & 3 of activation row 4 gi + (c >> 2); |acc| <= 2^15, exact in fp32
                const int sc = (c & 8) ? ((c & 4) ? S[3] : S[2]) : ((c & 4) ? S[1] : S[0]);
                const int e = 8 * (c & 3) - sc;
#pragma unroll
                for (int j = 0; j < 4; ++j) f[gi][j] += ldexpf((float)acc[j], e);
                __builtin_amdgcn_wave_barrier();   // the B reads are done before the next digits
            }
        }

        // the four digit columns of each activation row: the sum lands in lane c = 4 b + 3
#pragma unroll
        for (int gi = 0; gi < NG; ++gi)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float v = f[gi][j];
                v += dpp_f32<0x111>(v);   // row_shr:1
                v += dpp_f32<0x112>(v);   // row_shr:2
                f[gi][j] = v;
            }
        if ((c & 3) == 3) {
            float* dst = part + wave * NG * 64 + (c >> 2) * 16 + 4 * g;
#pragma unroll
            for (int gi = 0; gi < NG; ++gi)
#pragma unroll
                for (int j = 0; j < 4; ++j) dst[gi * 64 + j] = f[gi][j];
        }
        __syncthreads();
        for (int i = threadIdx.x; i < NG * 64; i += blockDim.x) {
            float sum = 0.f;
            for (int wv = 0; wv < nwaves; ++wv) sum += part[wv * NG * 64 + i];
            tot[i] = sum;
        }
        __syncthreads();
        // tot[b 16 + row] is the ternary row sum of activation row b; the row scale multiplies it once
        for (int i = threadIdx.x; i < 16 * batch; i += blockDim.x) {
            const int orow = tile * 16 + (i & 15);
            if (orow < n) y[(int64_t)(i >> 4) * n + orow] = scale[orow] * tot[i];
        }
    }
}

template <int NG>
hipError_t run_gemm(const uint32_t* packed, const float* scale, const float* x, float* y, int batch, int n,
                    int kq, hipStream_t stream) {
    const int waves = min(kMaxWaves, (kq + kSliceChunks - 1) / kSliceChunks);
    const size_t lds = gemm_lds_bytes(waves, NG);
    static int cache[kMaxWaves + 1] = {};   // resident workgroups per compute unit, per wave count
    if (cache[waves] == 0) {
        int per_cu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, ternary_gemm_kernel<NG>, kWave * waves, lds) !=
                hipSuccess ||
            per_cu < 1)
            per_cu = 1;
        cache[waves] = per_cu;
    }
    const int ntiles = (n + 15) / 16;
    const int grid = min(ntiles, cache[waves] * device_cu_count());
    ternary_gemm_kernel<NG><<<grid, kWave * waves, lds, stream>>>(packed, scale, x, y, batch, n, kq);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ternary_gemm(const uint32_t* packed, const float* row_scale, const float* x, float* y,
                               int64_t batch, int64_t n, int64_t k, hipStream_t stream) {
    const bool fast = k % 64 == 0 && (reinterpret_cast<uintptr_t>(packed) & 15u) == 0;
    if (!fast) {
        for (int64_t b = 0; b < batch; ++b) {
            const hipError_t e = launch_ternary(packed, row_scale, x + b * k, y + b * n, n, k, stream);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    const int nn = (int)n, kq = (int)(k / 64), bb = (int)batch;
    switch ((bb + 3) / 4) {
        case 1: return run_gemm<1>(packed, row_scale, x, y, bb, nn, kq, stream);
        case 2: return run_gemm<2>(packed, row_scale, x, y, bb, nn, kq, stream);
        case 3: return run_gemm<3>(packed, row_scale, x, y, bb, nn, kq, stream);
        default: return run_gemm<4>(packed, row_scale, x, y, bb, nn, kq, stream);
    }
}

}  // namespace e2m1
