// ternary_wl.hip -- widely-linear complex ternary GEMV (ternary_wl_gemv).
//
// Method: FairyFuse blog post, section "复杂值广泛线性层的融合核调度": a
// complex layer y = U x + W conj(x) whose matrices have ternary real and
// imaginary parts, evaluated as eight coupled real ternary GEMVs in one pass
// over the weights: each decoded weight serves both the real and the
// imaginary part of x (mask reuse), x is staged once for all eight (input
// reuse), the conjugate enters as a sign and never as a second copy of x, and
// the eight partial sums stay in registers until the final reduction. Each of
// U_re, U_im, W_re, W_im is packed like the real ternary GEMV (section
// "三元 GEMV 的乘法消除原理": 16 weights per word, bit 2j+1 = +1, bit 2j = -1)
// with its own per-row scale, applied once after the row sum.
//
// gfx950 design. The eight sub-GEMVs are a contraction of four ternary
// matrices against the same few columns of x, so the fast kernel runs them on
// the matrix cores: weights decode two at a time to bf16 +/-0.5 or 0 (a
// rotate, a mask and a v_perm_b32; the factor 2 goes into the scale) as the A
// operand of v_mfma_f32_16x16x32_bf16, and the B operand holds x_re and x_im,
// each split exactly into three bf16 pieces (hi = x truncated to bf16, mid =
// the remainder truncated, lo = what is left, at most 8 significant bits), in
// six of its sixteen columns. Products are exact and accumulate in fp32, so x
// is used at full fp32 precision. A dot2-based decode would need 32 dot
// products per 16-weight word against x_re and x_im (hi + lo each); here the
// matrix cores take that work and the vector ALU only decodes.
//
// Work split: a workgroup owns a tile of 16 rows; its waves split K into
// slices of 256 columns (lane l = 16 g + r loads the 16-byte chunk 4 s + g of
// row r of each matrix: four words, 64 columns). The matrix-core k-slots of a
// lane group are the columns of its chunk, in the order in which the pairs
// decode (fields p and p + 8 of word q), and the B operand of the same lanes
// lists x in that order, so the sum over k is complete whatever the order.
// D element (row 4 g + j, column c) sits in component j of lane 16 g + c. The
// three pieces of x_re (columns 0..2) and of x_im (3..5) are added by DPP
// within each 16-lane row, the slices through LDS, and one thread per row
// and component applies the four scales and the signs of the complex product.
// x is split into LDS once per workgroup when K fits one staged block (4096
// columns), else once per block and tile. Inputs the fast kernel cannot take
// (K % 64 != 0, unaligned matrices) use a one-wave-per-row kernel that adds,
// subtracts or skips each x directly.
#include "device.hpp"
#include "kernels.hpp"

namespace e2m1 {
namespace {

constexpr int kMaxWaves = 16;
constexpr int kSliceChunks = 4;                          // 64-column chunks per wave slice
constexpr int kVariants = 6;                             // x_re hi/mid/lo, x_im hi/mid/lo
constexpr int kRowDwords = 32;                           // bf16 pairs of one (chunk, variant)
constexpr int kRowPitch = 36;                            // dwords per row in LDS (spreads the banks)
constexpr int kPartFloats = 4 * 2 * 16;                  // (matrix, part, row) partial sums

struct WlMats {
    const uint32_t* m[4];   // U_re, U_im, W_re, W_im
};

__device__ __forceinline__ void issue_fence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// x = hi + mid + lo exactly: hi and mid are truncations to bf16, the rest
// has at most 8 significant bits and so is a bf16 value as well.
__device__ __forceinline__ void split3(float v, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
    const uint32_t h = __float_as_uint(v) & 0xFFFF0000u;
    const float r1 = v - __uint_as_float(h);
    const uint32_t m = __float_as_uint(r1) & 0xFFFF0000u;
    const float r2 = r1 - __uint_as_float(m);
    hi = h;
    mid = m;
    lo = __float_as_uint(r2);
}

// {a.high16, b.high16}: two bf16 pieces as one pair (a in the low half).
__device__ __forceinline__ uint32_t pair_hi16(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// Layout of the dynamic LDS of one workgroup with `bc` chunks per block.
struct WlLds {
    uint32_t* table;   // [bc][kVariants][kRowPitch]
    uint32_t* zero;    // kRowDwords zeros (B columns 6..15)
    float* part;       // [waves][kPartFloats]
    float* tot;        // [kPartFloats]
};

__device__ __forceinline__ WlLds wl_lds(uint32_t* base, int bc, int waves) {
    WlLds l;
    l.table = base;
    l.zero = base + bc * kVariants * kRowPitch;
    l.part = reinterpret_cast<float*>(l.zero + kRowDwords);
    l.tot = l.part + waves * kPartFloats;
    return l;
}

size_t wl_lds_bytes(int bc, int waves) {
    return 4u * ((size_t)bc * kVariants * kRowPitch + kRowDwords + (size_t)waves * kPartFloats + kPartFloats);
}

// Pair slot s of block chunk `cl`: columns k0 = 64 c + 16 q + 4 h + d and
// k0 + 8 with (q, h, d) = (s >> 3 & 3, s >> 2 & 1, s & 3): the two fields that
// one perm decodes (p = 4 h + d and p + 8 of word q).
__device__ __forceinline__ int slot_column(int chunk, int s) {
    return 64 * chunk + 16 * ((s >> 3) & 3) + 4 * ((s >> 2) & 1) + (s & 3);
}

struct XSlot {
    float r0, r1, i0, i1;
};

__device__ __forceinline__ XSlot load_slot(const float* x_re, const float* x_im, int chunk, int s, int K) {
    const int k0 = min(slot_column(chunk, s), K - 1);
    const int k1 = min(k0 + 8, K - 1);
    return XSlot{x_re[k0], x_re[k1], x_im[k0], x_im[k1]};
}

__device__ __forceinline__ void store_slot(uint32_t* table, int cl, int s, const XSlot& v) {
    uint32_t h0, m0, l0, h1, m1, l1;
    uint32_t* row = table + cl * kVariants * kRowPitch + (s & 31);
    split3(v.r0, h0, m0, l0);
    split3(v.r1, h1, m1, l1);
    row[0 * kRowPitch] = pair_hi16(h0, h1);
    row[1 * kRowPitch] = pair_hi16(m0, m1);
    row[2 * kRowPitch] = pair_hi16(l0, l1);
    split3(v.i0, h0, m0, l0);
    split3(v.i1, h1, m1, l1);
    row[3 * kRowPitch] = pair_hi16(h0, h1);
    row[4 * kRowPitch] = pair_hi16(m0, m1);
    row[5 * kRowPitch] = pair_hi16(l0, l1);
}

// A operand for MFMA (q, h): fields 4 h .. 4 h + 3 of word q and the fields 8 above them.
template <int H>
__device__ __forceinline__ u32x4 decode_half(uint32_t w) {
    u32x4 a;
    a.x = ternary_pair<4 * H + 0>(w);
    a.y = ternary_pair<4 * H + 1>(w);
    a.z = ternary_pair<4 * H + 2>(w);
    a.w = ternary_pair<4 * H + 3>(w);
    return a;
}

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
}

// One wave slice: four weight chunks (one per matrix) against the B operands of the chunk.
__device__ __forceinline__ void slice_mfma(const uint4 (&w)[4], uint32_t mask, const u32x4 (&b)[8], f32x4 (&acc)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint32_t ws[4] = {w[m].x, w[m].y, w[m].z, w[m].w};
            const uint32_t word = ws[q] & mask;
            acc[m] = mfma_bf16(decode_half<0>(word), b[2 * q + 0], acc[m]);
            acc[m] = mfma_bf16(decode_half<1>(word), b[2 * q + 1], acc[m]);
        }
    }
}

__device__ __forceinline__ void load_b(const uint32_t* src, u32x4 (&b)[8]) {
    const u32x4* p = reinterpret_cast<const u32x4*>(src);
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = p[i];
}

// Row totals of one tile: DPP sums of the x pieces, LDS sums over the waves,
// then scales and the signs of the complex product; writes y_re, y_im.
__device__ __forceinline__ void tile_epilogue(const f32x4 (&acc)[4], const WlLds& l, int wave, int nwaves,
                                              int lane, const float (&sc)[4], float* y_re, float* y_im,
                                              int tile, int n) {
    const int g = lane >> 4, c = lane & 15;
    float s[4][4];   // lane c: D(c) + D(c - 1) + D(c - 2) within its 16-lane row
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float v = acc[m][j];
            s[m][j] = v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xF, 0xF, true)) +
                      __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xF, 0xF, true));
        }
    }
    if (c == 2 || c == 5) {   // x_re pieces (columns 0..2), x_im pieces (3..5)
        float* dst = l.part + wave * kPartFloats + (c == 5 ? 16 : 0) + 4 * g;
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j) dst[32 * m + j] = s[m][j];
    }
    __syncthreads();
    const int t = threadIdx.x;
    for (int i = t; i < kPartFloats; i += blockDim.x) {   // one-wave workgroups take two rounds
        float sum = 0.f;
        for (int w = 0; w < nwaves; ++w) sum += l.part[w * kPartFloats + i];
        l.tot[i] = sum;
    }
    __syncthreads();
    if (t < 32) {
        const int r = t & 15, row = tile * 16 + r;
        // P(m, part) = half the ternary row sum of matrix m against x_part
        const float* P = l.tot;
        const float ur_re = P[0 * 16 + r], ur_im = P[1 * 16 + r], ui_re = P[2 * 16 + r], ui_im = P[3 * 16 + r];
        const float wr_re = P[4 * 16 + r], wr_im = P[5 * 16 + r], wi_re = P[6 * 16 + r], wi_im = P[7 * 16 + r];
        float y;
        if (t < 16)   // Re: U_re x_re - U_im x_im + W_re x_re + W_im x_im
            y = (sc[0] * (2.f * ur_re) - sc[1] * (2.f * ui_im)) + (sc[2] * (2.f * wr_re) + sc[3] * (2.f * wi_im));
        else          // Im: U_re x_im + U_im x_re - W_re x_im + W_im x_re
            y = (sc[0] * (2.f * ur_im) + sc[1] * (2.f * ui_re)) + (sc[3] * (2.f * wi_re) - sc[2] * (2.f * wr_im));
        if (row < n) (t < 16 ? y_re : y_im)[row] = y;
    }
}

// Fast kernel: K % 64 == 0, matrices 16-byte aligned. kOneBlock: all of K
// fits one staged block of 4 * waves chunks, so x is split once per
// workgroup and each wave keeps its B operands in registers across tiles.
template <bool kOneBlock>
__global__ __launch_bounds__(kWave * kMaxWaves) void ternary_wl_kernel(WlMats mats, const float* scale,
                                                                       const float* x_re, const float* x_im,
                                                                       float* y_re, float* y_im, int n, int kq) {
    extern __shared__ __attribute__((aligned(16))) uint32_t wl_smem[];
    const int nwaves = blockDim.x / kWave;
    const int bc = kSliceChunks * nwaves;
    const WlLds l = wl_lds(wl_smem, bc, nwaves);
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int g = lane >> 4, r = lane & 15, c = lane & 15;
    const int K = 64 * kq;
    const int ntiles = (n + 15) / 16;
    const int nblocks = (kq + bc - 1) / bc;

    if (threadIdx.x < kRowDwords) l.zero[threadIdx.x] = 0u;

    for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int row = min(tile * 16 + r, n - 1);
        float sc[4] = {0.f, 0.f, 0.f, 0.f};
        if (wave == 0) {
#pragma unroll
            for (int m = 0; m < 4; ++m) sc[m] = scale[(int64_t)m * n + row];
        }
        f32x4 acc[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int blk = 0; blk < nblocks; ++blk) {
            const int chunk = blk * bc + wave * kSliceChunks + g;
            const int cc = min(chunk, kq - 1);
            const uint32_t mask = chunk < kq ? 0xFFFFFFFFu : 0u;
            const bool split = !kOneBlock || tile == (int)blockIdx.x;
            XSlot xs[2];
            if (split) {
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int s = threadIdx.x + i * blockDim.x;
                    xs[i] = load_slot(x_re, x_im, blk * bc + (s >> 5), s, K);
                }
            }
            issue_fence();
            uint4 w[4];
#pragma unroll
            for (int m = 0; m < 4; ++m)
                w[m] = load_nt16(mats.m[m] + ((int64_t)row * kq + cc) * 4);
            issue_fence();
            if (split) {
                if (!kOneBlock) __syncthreads();   // the previous block's B reads are done
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int s = threadIdx.x + i * blockDim.x;
                    store_slot(l.table, s >> 5, s, xs[i]);
                }
                __syncthreads();
            }
            u32x4 b[8];
            const int cl = cc - blk * bc;
            load_b(c < kVariants ? l.table + (cl * kVariants + c) * kRowPitch : l.zero, b);
            slice_mfma(w, mask, b, acc);
        }
        tile_epilogue(acc, l, wave, nwaves, lane, sc, y_re, y_im, tile, n);
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

struct WlConfig {
    int waves;
    size_t lds;
    int resident;   // workgroups per compute unit
};

template <bool kOneBlock>
int wl_resident(int waves, size_t lds) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, ternary_wl_kernel<kOneBlock>, kWave * waves, lds) !=
            hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    return per_cu;
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
        const int bc = kSliceChunks * waves;
        const bool one = kq <= bc;
        const size_t lds = wl_lds_bytes(bc, waves);
        // resident workgroups per compute unit, per (wave count, variant)
        static int cache[2][kMaxWaves + 1] = {};
        int& per_cu = cache[one][waves];
        if (per_cu == 0) per_cu = one ? wl_resident<true>(waves, lds) : wl_resident<false>(waves, lds);
        const int ntiles = (nn + 15) / 16;
        const int grid = min(ntiles, per_cu * device_cu_count());
        if (one)
            ternary_wl_kernel<true><<<grid, kWave * waves, lds, stream>>>(wm, scale, x_re, x_im, y_re, y_im, nn, kq);
        else
            ternary_wl_kernel<false><<<grid, kWave * waves, lds, stream>>>(wm, scale, x_re, x_im, y_re, y_im, nn, kq);
        return hipGetLastError();
    }
    const int want = (nn + 3) / 4;
    const int grid = min(want, 8 * device_cu_count());
    ternary_wl_generic_kernel<<<grid, 256, 0, stream>>>(wm, scale, x_re, x_im, y_re, y_im, nn, (int)(k / 16));
    return hipGetLastError();
}

}  // namespace e2m1
