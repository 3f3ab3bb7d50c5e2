// ternary_batch.hip -- small-batch ternary GEMM (ternary_gemm).
//
// Method: the ternary GEMV of the FairyFuse blog post (section
// "三元 GEMV 的乘法消除原理": 16 weights per word, bit 2j+1 = +1, bit 2j = -1,
// the per-row scale applied once after the row sum) for a few activation rows
// at once; section "总结与启示" names this batched fusion for speculative
// decoding as the next step. Every weight is decoded once for all rows.
//
// gfx950 design: the int8 matrix-core formulation of ternary_int8.hpp. Each
// group of two activation rows fills the sixteen B columns of one
// v_mfma_i32_16x16x64_i8 (row 2 gi + b of group gi in columns 8 b .. 8 b + 7:
// the four base-256 digits of its integer part, then those of its fraction),
// so a decoded A operand serves ceil(batch / 2) MFMAs; the int32 sums are
// exact and each digit column is scaled into fp32 per 256-column slice. A
// workgroup owns a tile of 16 output rows (one workgroup per tile) and its
// waves take 256-column slices; lane l = 16 g + r loads the 16-byte chunk 4 s + g of row r (four
// words) and decodes word q as the A operand of one MFMA per group. Each wave
// writes the digits of its own slice into its own LDS area (lane l: columns
// 16 q + j + 4 b of chunk l >> 4, word l >> 2 & 3, dword j = l & 3, b = 0..3,
// of every row of the group) and reads them back as B operands, with no
// workgroup barrier. D element (output row 4 g + j, column c) is component j
// of lane 16 g + c; the eight digit columns of each activation row are added
// by DPP, the waves through LDS (one barrier), and the row scale multiplies
// the total once.
// Every workgroup prepares the digits of every activation row this way, so
// their VALU work (about 225 instructions per group of two rows per wave)
// grows with the batch in each of the n / 16 tiles. From five rows on the
// digits are instead prepared once per call by a launch of their own into the
// caller's workspace, already in the B-operand layout, and the GEMM loads them
// (1 KB contiguous per instruction) and does no digit arithmetic; there each
// wave serves two 16-row tiles and the two halves of the slices run in
// workgroups of their own, each adding its share into y (zeroed by the
// pre-pass; two addends onto zero, so the result does not depend on their
// order).
// Inputs the fast kernels cannot take (K % 64 != 0, unaligned weights) run the
// ternary GEMV once per activation row.
#include "device.hpp"
#include "kernels.hpp"
#include "ternary_int8.hpp"

namespace e2m1 {
namespace {

constexpr int kMaxWaves = 16;
constexpr int kSliceChunks = 4;                               // 64-column chunks per wave slice
constexpr int kColumns = 16;                                  // B columns: 2 rows x 8 digits
constexpr int kGroupRows = 2;                                 // activation rows per MFMA
constexpr int kRowPitch = 20;                                 // dwords per (chunk, column) row in LDS
// dwords per chunk: 16 more than its 16 rows, so the four chunks' rows start 16 banks apart and the
// digit writes of a wave (one dword per lane, the four chunks side by side) meet no bank twice
constexpr int kChunkPitch = kColumns * kRowPitch + 16;
constexpr int kWaveDwords = kSliceChunks * kChunkPitch;
// From this batch on the digits are prepared once per call (4096 x 4096, event us, one launch against
// two: B = 4 6.17 / 6.6 (estimated from B = 6 and 8), B = 6 7.97 / 7.16, B = 8 9.7 / 7.74, B = 16
// 16.4 / 10.28): the pre-pass is a launch of a few µs, and the GEMM then reads 8 bytes of digits per
// activation element for every two tiles.
constexpr int kPrepassMinBatch = 5;
constexpr int kPreWaves = 8;                                  // waves per workgroup of the two-launch GEMM

size_t gemm_lds_bytes(int waves, int groups) {
    return 4u * ((size_t)waves * kWaveDwords + (size_t)waves * groups * 32);
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
    float* part = reinterpret_cast<float*>(tg_smem + nwaves * kWaveDwords);   // [waves][NG * 2 rows][16]
    const int g = lane >> 4, r = lane & 15, c = lane & 15;
    const int K = 64 * kq;
    const int nslices = (kq + kSliceChunks - 1) / kSliceChunks;
    // digit preparation: lane -> chunk pg, word pq, dword pj; columns 64 pg + 16 pq + pj + 4 b
    const int pg = lane >> 4, pq = (lane >> 2) & 3, pj = lane & 3;
    uint32_t* prep_row = tab + pg * kChunkPitch + 4 * pq + pj;
    const i32x4* b_row = reinterpret_cast<const i32x4*>(tab + g * kChunkPitch + c * kRowPitch);
    // digit column c: activation row c >> 3 of the group, fraction digits for c & 4, digit c & 3
    const int c_row = c >> 3, c_shift = 8 * (c & 3) - ((c & 4) ? 30 : 0);
    const int tile = blockIdx.x;   // one tile of 16 output rows per workgroup
    const int row = min(tile * 16 + r, n - 1);
    float f[NG][4];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi)
#pragma unroll
        for (int j = 0; j < 4; ++j) f[gi][j] = 0.f;

    // every activation row of the slice is kept in registers, requested before the weights (this
    // form runs up to three groups)
    for (int sl = wave; sl < nslices; sl += nwaves) {   // wave-uniform
        const int col0 = 256 * sl + 64 * pg + 16 * pq + pj;
        float xa[NG][kGroupRows][4];   // [group][row of the group][b]
#pragma unroll
        for (int ga = 0; ga < NG; ++ga)
#pragma unroll
            for (int bl = 0; bl < kGroupRows; ++bl) {
                const int b_row_x = min(kGroupRows * ga + bl, batch - 1);   // rows past the batch: never prepared
                const float* xr = x + (int64_t)b_row_x * K;
#pragma unroll
                for (int b = 0; b < 4; ++b) xa[ga][bl][b] = xr[min(col0 + 4 * b, K - 1)];
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
            const int rows = min(kGroupRows, batch - kGroupRows * gi);   // rows of this group (uniform, >= 1)
            float xv[kGroupRows][4];
#pragma unroll
            for (int bl = 0; bl < kGroupRows; ++bl)
#pragma unroll
                for (int b = 0; b < 4; ++b) xv[bl][b] = xa[gi][bl][b];
            // digit columns of rows past the batch keep whatever integers LDS holds: their
            // D columns are never read
            int S[kGroupRows] = {30, 30};
#pragma unroll
            for (int bl = 0; bl < kGroupRows; ++bl) {
                if (bl >= rows) break;
                S[bl] = slice_exponent(wave_max(fmaxf(fmaxf(fabsf(xv[bl][0]), fabsf(xv[bl][1])),
                                                      fmaxf(fabsf(xv[bl][2]), fabsf(xv[bl][3])))));
                uint32_t dh[4], dl[4], th[4], tl[4];
#pragma unroll
                for (int b = 0; b < 4; ++b) digits8(xv[bl][b], S[bl], dh[b], dl[b]);
                transpose4(dh, th);
                transpose4(dl, tl);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    prep_row[(8 * bl + i) * kRowPitch] = th[i];
                    prep_row[(8 * bl + 4 + i) * kRowPitch] = tl[i];
                }
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
            // |acc| <= 256 * 128: exact in fp32
            const int e = c_shift - (c_row ? S[1] : S[0]);
#pragma unroll
            for (int j = 0; j < 4; ++j) f[gi][j] += ldexpf((float)acc[j], e);
            __builtin_amdgcn_wave_barrier();   // the B reads are done before the next digits
        }
    }

    // the eight digit columns of each activation row: the sum lands in lane c = 8 b + 7
#pragma unroll
    for (int gi = 0; gi < NG; ++gi)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float v = f[gi][j];
            v += dpp_f32<0x111>(v);   // row_shr:1
            v += dpp_f32<0x112>(v);   // row_shr:2
            v += dpp_f32<0x114>(v);   // row_shr:4
            f[gi][j] = v;
        }
    if ((c & 7) == 7) {
        float* dst = part + wave * NG * 32 + c_row * 16 + 4 * g;
#pragma unroll
        for (int gi = 0; gi < NG; ++gi)
#pragma unroll
            for (int j = 0; j < 4; ++j) dst[gi * 32 + j] = f[gi][j];
    }
    __syncthreads();
    // part[wave][b 16 + row] holds the wave's share of activation row b; summed over the waves in
    // a fixed order, then the row scale multiplies the total once
    for (int i = threadIdx.x; i < 16 * batch; i += blockDim.x) {
        const int orow = tile * 16 + (i & 15);
        float sum = 0.f;
        for (int wv = 0; wv < nwaves; ++wv) sum += part[wv * NG * 32 + i];
        if (orow < n) y[(int64_t)(i >> 4) * n + orow] = scale[orow] * sum;
    }
}

// Two-launch form (batch >= kPrepassMinBatch): the digits above depend only
// on x, so ternary_digits_kernel prepares them once per launch instead of once per tile. One wave
// per (group gi of two activation rows, 256-column slice sl) computes them exactly as above and
// stores them already in the B-operand layout: operand q of lane l for (gi, sl) is the 16 bytes
// at ((gi * nslices + sl) * 4 + q) * 1024 + 16 l of the digit area, so the GEMM's loads read
// 1 KB contiguous per instruction; the exponent S of activation row b and slice sl follows at
// [b][sl]. Rows past the batch get zero digits and S = 30.
__global__ __launch_bounds__(kWave) void ternary_digits_kernel(const float* __restrict__ x,
                                                               uint32_t* __restrict__ dig,
                                                               int* __restrict__ sexp, float* __restrict__ y,
                                                               int batch, int n, int kq) {
    const int sl = blockIdx.x, gi = blockIdx.y, nslices = gridDim.x;
    const int lane = threadIdx.x;
    // y starts at zero: the GEMM's two K halves each add their share
    const int64_t ny = (int64_t)batch * n, nthreads = (int64_t)kWave * nslices * gridDim.y;
    for (int64_t i = ((int64_t)gi * nslices + sl) * kWave + lane; i < ny; i += nthreads) y[i] = 0.f;
    const int K = 64 * kq;
    const int pg = lane >> 4, pq = (lane >> 2) & 3, pj = lane & 3;
    const int col0 = 256 * sl + 64 * pg + 16 * pq + pj;
    float xv[kGroupRows][4];
#pragma unroll
    for (int bl = 0; bl < kGroupRows; ++bl) {
        const float* xr = x + (int64_t)min(kGroupRows * gi + bl, batch - 1) * K;
#pragma unroll
        for (int b = 0; b < 4; ++b) xv[bl][b] = xr[min(col0 + 4 * b, K - 1)];
    }
    // dword 4 pq + pj of row (chunk pg, digit column c): operand pq of lane 16 pg + c, dword pj
    uint32_t* dst = dig + ((int64_t)(gi * nslices + sl) * 4 + pq) * 256 + 16 * 4 * pg + pj;
#pragma unroll
    for (int bl = 0; bl < kGroupRows; ++bl) {
        const bool live = kGroupRows * gi + bl < batch;   // wave-uniform
        const int S = live ? slice_exponent(wave_max(fmaxf(fmaxf(fabsf(xv[bl][0]), fabsf(xv[bl][1])),
                                                           fmaxf(fabsf(xv[bl][2]), fabsf(xv[bl][3])))))
                           : 30;
        uint32_t dh[4], dl[4], th[4], tl[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) digits8(xv[bl][b], S, dh[b], dl[b]);
        transpose4(dh, th);
        transpose4(dl, tl);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            dst[(8 * bl + i) * 4] = live ? th[i] : 0u;
            dst[(8 * bl + 4 + i) * 4] = live ? tl[i] : 0u;
        }
        if (lane == 0) sexp[(int64_t)(kGroupRows * gi + bl) * nslices + sl] = S;
    }
}

// The GEMM of the two-launch form: the slice and MFMA structure of ternary_gemm_kernel, with
// each group's four B operands and two exponents loaded (group gi + 1's requested before group
// gi's products) instead of prepared. Each wave takes two 16-row tiles (rows 32 blockIdx.x + 16 t
// + r), so every loaded operand serves two MFMAs, and the workgroups of blockIdx.y = 0 and 1 take
// the first and the second half of the slices (256 workgroups at n = 4096). Each half adds
// fl(scale * its sum over its waves) into y, which the pre-pass zeroed: with exactly two addends
// onto zero the result does not depend on their order (0 + a = a, a + b = b + a).
template <int NG>
__global__ __launch_bounds__(kWave * kPreWaves) void ternary_gemm_pre_kernel(const uint32_t* packed,
                                                                             const float* scale,
                                                                             const uint32_t* dig,
                                                                             const int* sexp, float* y,
                                                                             int batch, int n, int kq) {
    extern __shared__ __attribute__((aligned(16))) float tp_part[];   // [waves][NG][2 tiles][2 rows][16]
    const int nwaves = blockDim.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int g = lane >> 4, r = lane & 15, c = lane & 15;
    const int nslices = (kq + kSliceChunks - 1) / kSliceChunks;
    const int half = (nslices + 1) / 2;
    const int sl0 = blockIdx.y * half, sl1 = min(nslices, sl0 + half);
    const int c_row = c >> 3, c_shift = 8 * (c & 3) - ((c & 4) ? 30 : 0);
    const int rows0 = blockIdx.x * 32;
    int64_t rbase[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) rbase[t] = (int64_t)min(rows0 + 16 * t + r, n - 1) * kq;
    float f[NG][2][4];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) f[gi][t][j] = 0.f;
    for (int sl = sl0 + wave; sl < sl1; sl += nwaves) {   // wave-uniform
        const i32x4* ops = reinterpret_cast<const i32x4*>(dig) + (int64_t)sl * 4 * 64 + lane;
        const int* se = sexp + (int64_t)c_row * nslices + sl;
        const int64_t gstride = (int64_t)nslices * 4 * 64;   // i32x4 per group
        i32x4 bq[2][4];
        int sv[2];
#pragma unroll
        for (int q = 0; q < 4; ++q) bq[0][q] = ops[q * 64];
        sv[0] = se[0];
        issue_fence();
        const int chunk = sl * kSliceChunks + g;
        const uint32_t mask = chunk < kq ? 0xFFFFFFFFu : 0u;
        uint4 w[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) w[t] = load_nt16(packed + (rbase[t] + min(chunk, kq - 1)) * 4);
        issue_fence();
        i32x4 a[2][4];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            if (gi + 1 < NG) {
#pragma unroll
                for (int q = 0; q < 4; ++q) bq[(gi + 1) & 1][q] = ops[(gi + 1) * gstride + q * 64];
                sv[(gi + 1) & 1] = se[(int64_t)(gi + 1) * kGroupRows * nslices];
                issue_fence();
            }
            if (gi == 0) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const uint32_t ws[4] = {w[t].x & mask, w[t].y & mask, w[t].z & mask, w[t].w & mask};
#pragma unroll
                    for (int q = 0; q < 4; ++q) a[t][q] = decode_word(ws[q]);
                }
            }
            const int e = c_shift - sv[gi & 1];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                i32x4 acc = {0, 0, 0, 0};
#pragma unroll
                for (int q = 0; q < 4; ++q) acc = mfma_i8(a[t][q], bq[gi & 1][q], acc);
#pragma unroll
                for (int j = 0; j < 4; ++j) f[gi][t][j] += ldexpf((float)acc[j], e);
            }
        }
    }
    // the eight digit columns of each activation row: lane (g, c) ends with the totals of values
    // (c & 7) NG + m of the flattened [gi][t][j] (NG of them)
    float v[NG * 8];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) v[(gi * 2 + t) * 4 + j] = f[gi][t][j];
    digit_lane_totals(v, lane);
    {
        float* dst = tp_part + wave * NG * 64 + c_row * 16 + 4 * g;
#pragma unroll
        for (int m = 0; m < NG; ++m) {
            const int fi = (c & 7) * NG + m, gi = fi >> 3, t = (fi >> 2) & 1, j = fi & 3;
            dst[gi * 64 + t * 32 + j] = v[m];
        }
    }
    __syncthreads();
    // o = (activation row b, tile t, row i): b = 2 gi + c_row
    for (int o = threadIdx.x; o < 32 * batch; o += blockDim.x) {
        const int b = o >> 5, t = (o >> 4) & 1, i = o & 15;
        const int orow = rows0 + 16 * t + i;
        const int idx = (b >> 1) * 64 + t * 32 + (b & 1) * 16 + i;
        float sum = 0.f;
        for (int wv = 0; wv < nwaves; ++wv) sum += tp_part[wv * NG * 64 + idx];
        if (orow < n) atomicAdd(y + (int64_t)b * n + orow, scale[orow] * sum);
    }
}

// Batch 1 (ternary_gemv): the kernel above with one activation row, and each
// wave's SPW slices (slice wave + waves i) known at compile time, so the x
// and weight loads of all of them are issued before the first is used.
template <int SPW>
__global__ __launch_bounds__(kWave * kMaxWaves) void ternary_gemv_i8_kernel(const uint32_t* packed,
                                                                            const float* scale, const float* x,
                                                                            float* y, int n, int kq) {
    extern __shared__ __attribute__((aligned(16))) uint32_t tv_smem[];
    const int nwaves = blockDim.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    uint32_t* tab = tv_smem + wave * kWaveDwords;
    float* part = reinterpret_cast<float*>(tv_smem + nwaves * kWaveDwords);   // [waves][16]
    const int g = lane >> 4, r = lane & 15, c = lane & 15;
    const int K = 64 * kq;
    const int nslices = (kq + kSliceChunks - 1) / kSliceChunks;
    const int pg = lane >> 4, pq = (lane >> 2) & 3, pj = lane & 3;
    uint32_t* prep_row = tab + pg * kChunkPitch + 4 * pq + pj;
    const i32x4* b_row = reinterpret_cast<const i32x4*>(tab + g * kChunkPitch + c * kRowPitch);
    const int c_shift = 8 * (c & 3) - ((c & 4) ? 30 : 0);   // columns 0..7: the row's eight digits
    const int tile = blockIdx.x;
    const int row = min(tile * 16 + r, n - 1);
    float xv[SPW][4];
    uint4 w[SPW];
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int col0 = 256 * min(wave + nwaves * i, nslices - 1) + 64 * pg + 16 * pq + pj;
#pragma unroll
        for (int b = 0; b < 4; ++b) xv[i][b] = x[min(col0 + 4 * b, K - 1)];
    }
    issue_fence();
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int chunk = (wave + nwaves * i) * kSliceChunks + g;
        w[i] = load_nt16(packed + ((int64_t)row * kq + min(chunk, kq - 1)) * 4);
    }
    issue_fence();
    float f[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int sl = wave + nwaves * i;
        if (sl >= nslices) break;   // wave-uniform
        const int S = slice_exponent(wave_max(fmaxf(fmaxf(fabsf(xv[i][0]), fabsf(xv[i][1])),
                                                    fmaxf(fabsf(xv[i][2]), fabsf(xv[i][3])))));
        uint32_t dh[4], dl[4], th[4], tl[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) digits8(xv[i][b], S, dh[b], dl[b]);
        transpose4(dh, th);
        transpose4(dl, tl);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            prep_row[q * kRowPitch] = th[q];
            prep_row[(4 + q) * kRowPitch] = tl[q];
        }
        __builtin_amdgcn_wave_barrier();   // LDS accesses of one wave complete in order
        const int chunk = sl * kSliceChunks + g;
        const uint32_t mask = chunk < kq ? 0xFFFFFFFFu : 0u;
        const uint32_t ws[4] = {w[i].x & mask, w[i].y & mask, w[i].z & mask, w[i].w & mask};
        i32x4 acc = {0, 0, 0, 0};
#pragma unroll
        for (int q = 0; q < 4; ++q) acc = mfma_i8(decode_word(ws[q]), b_row[q], acc);
        const int e = c_shift - S;   // columns 8..15 hold stale integers and are never read
#pragma unroll
        for (int j = 0; j < 4; ++j) f[j] += ldexpf((float)acc[j], e);
        __builtin_amdgcn_wave_barrier();   // the B reads are done before the next digits
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {   // the eight digit columns: the sum lands in lane c = 7
        float v = f[j];
        v += dpp_f32<0x111>(v);   // row_shr:1
        v += dpp_f32<0x112>(v);   // row_shr:2
        v += dpp_f32<0x114>(v);   // row_shr:4
        f[j] = v;
    }
    if (c == 7) {
#pragma unroll
        for (int j = 0; j < 4; ++j) part[wave * 16 + 4 * g + j] = f[j];
    }
    __syncthreads();
    if (threadIdx.x < 16) {
        float sum = 0.f;
        for (int wv = 0; wv < nwaves; ++wv) sum += part[wv * 16 + threadIdx.x];
        const int orow = tile * 16 + threadIdx.x;
        if (orow < n) y[orow] = scale[orow] * sum;
    }
}

template <int SPW>
hipError_t run_gemv_i8(const uint32_t* packed, const float* scale, const float* x, float* y, int n, int kq,
                       hipStream_t stream) {
    const int waves = min(kMaxWaves, (kq + kSliceChunks - 1) / kSliceChunks);
    const size_t lds = 4u * ((size_t)waves * kWaveDwords + (size_t)waves * 16);
    ternary_gemv_i8_kernel<SPW><<<(n + 15) / 16, kWave * waves, lds, stream>>>(packed, scale, x, y, n, kq);
    return hipGetLastError();
}

static_assert(kPrepassMinBatch % 2 == 1, "a group of two rows never straddles the two forms");

template <int NG>
hipError_t run_gemm(const uint32_t* packed, const float* scale, const float* x, float* y, int batch, int n,
                    int kq, void* workspace, hipStream_t stream) {
    const int nslices = (kq + kSliceChunks - 1) / kSliceChunks;
    const int waves = min(kMaxWaves, nslices);
    const int ntiles = (n + 15) / 16;   // one workgroup per tile: the hardware streams through them
    if constexpr (2 * NG > kPrepassMinBatch) {   // every batch of NG groups is >= kPrepassMinBatch
        if (workspace == nullptr) return hipErrorInvalidValue;
        uint32_t* dig = static_cast<uint32_t*>(workspace);
        int* sexp = reinterpret_cast<int*>(dig + (size_t)NG * nslices * 1024);
        ternary_digits_kernel<<<dim3(nslices, NG), kWave, 0, stream>>>(x, dig, sexp, y, batch, n, kq);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int pwaves = min(kPreWaves, (nslices + 1) / 2);
        ternary_gemm_pre_kernel<NG><<<dim3((n + 31) / 32, 2), kWave * pwaves, 4u * (size_t)pwaves * NG * 64,
                                      stream>>>(packed, scale, dig, sexp, y, batch, n, kq);
        return hipGetLastError();
    } else {
        const size_t lds = gemm_lds_bytes(waves, NG);
        ternary_gemm_kernel<NG><<<ntiles, kWave * waves, lds, stream>>>(packed, scale, x, y, batch, n, kq);
        return hipGetLastError();
    }
}

}  // namespace

size_t ternary_gemm_workspace_bytes(int64_t batch, int64_t k) {
    if (batch < kPrepassMinBatch || k % 64 != 0) return 0;
    const int64_t groups = (batch + kGroupRows - 1) / kGroupRows;
    const int64_t nslices = (k / 64 + kSliceChunks - 1) / kSliceChunks;
    return (size_t)(groups * nslices) * (4096 + 4 * kGroupRows);
}

hipError_t launch_ternary_gemm(const uint32_t* packed, const float* row_scale, const float* x, float* y,
                               int64_t batch, int64_t n, int64_t k, void* workspace, hipStream_t stream) {
    const bool fast = k % 64 == 0 && (reinterpret_cast<uintptr_t>(packed) & 15u) == 0;
    if (!fast) {
        for (int64_t b = 0; b < batch; ++b) {
            const hipError_t e = launch_ternary(packed, row_scale, x + b * k, y + b * n, n, k, stream);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    const int nn = (int)n, kq = (int)(k / 64), bb = (int)batch;
    const int nslices = (kq + kSliceChunks - 1) / kSliceChunks;
    if (bb == 1 && nslices <= 4 * kMaxWaves) {   // slices per wave known at compile time
        switch ((nslices + kMaxWaves - 1) / kMaxWaves) {
            case 1: return run_gemv_i8<1>(packed, row_scale, x, y, nn, kq, stream);
            case 2: return run_gemv_i8<2>(packed, row_scale, x, y, nn, kq, stream);
            case 3: return run_gemv_i8<3>(packed, row_scale, x, y, nn, kq, stream);
            default: return run_gemv_i8<4>(packed, row_scale, x, y, nn, kq, stream);
        }
    }
    switch ((bb + kGroupRows - 1) / kGroupRows) {
        case 1: return run_gemm<1>(packed, row_scale, x, y, bb, nn, kq, workspace, stream);
        case 2: return run_gemm<2>(packed, row_scale, x, y, bb, nn, kq, workspace, stream);
        case 3: return run_gemm<3>(packed, row_scale, x, y, bb, nn, kq, workspace, stream);
        case 4: return run_gemm<4>(packed, row_scale, x, y, bb, nn, kq, workspace, stream);
        case 5: return run_gemm<5>(packed, row_scale, x, y, bb, nn, kq, workspace, stream);
        case 6: return run_gemm<6>(packed, row_scale, x, y, bb, nn, kq, workspace, stream);
        case 7: return run_gemm<7>(packed, row_scale, x, y, bb, nn, kq, workspace, stream);
        default: return run_gemm<8>(packed, row_scale, x, y, bb, nn, kq, workspace, stream);
    }
}

}  // namespace e2m1
