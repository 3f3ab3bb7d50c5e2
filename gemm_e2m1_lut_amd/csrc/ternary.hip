// ternary.hip -- 2-bit ternary GEMV (ternary_gemv).
//
// Method: FairyFuse blog post, section "三元 GEMV 的乘法消除原理": 16 weights
// per 32-bit word; weight j of word w multiplies x[16w + j]; bit 2j+1 set
// adds x, bit 2j set subtracts x, neither contributes nothing; the per-row
// scale is the only multiply and is applied once, after the row sum.
//
// gfx950 design. The page's CPU kernel extracts +1/-1 lane masks with BMI2
// pext so that AVX-512 masked adds can use them. A GPU has no pext and a
// per-field compare-and-select costs about six VALU operations per weight, so
// the fast kernel decodes two fields at a time instead: a rotate and a mask
// turn them into a v_perm_b32 selector that looks up bf16 +0.5 / -0.5 / 0,
// and v_dot2_f32_bf16 accumulates the pair against x held as bf16 hi + lo
// parts (x = hi + lo to a relative 2^-16), about 2.5 operations per weight;
// the exact factor 2 goes into the row scale. Each lane owns one 64-column
// chunk of K (one 16-byte load of four words); lanes cover a row in groups
// (64 lanes for K = 4096, fewer for short rows) and the row total comes from
// a DPP-only reduction, multiplied by the row scale once. The hi/lo split of
// x is done once per workgroup of 16 waves into LDS (a few operations per
// thread) rather than once per wave, and every weight load is issued before
// the split so that its latency is hidden behind it. Inputs the fast kernel
// cannot take (K % 64 != 0, K > 4096, unaligned pointers) use a
// one-wave-per-row kernel that adds, subtracts or skips each x directly.
#include "device.hpp"
#include "kernels.hpp"

namespace e2m1 {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;

// Row total of groups of G lanes (G in {8, 16, 32, 64}) with DPP only: the
// total ends up in the last lane of each group.
template <int G>
__device__ __forceinline__ float group_total(float v) {
    v += dpp_f32<0xB1>(v);
    v += dpp_f32<0x4E>(v);
    v += dpp_f32<0x141>(v);
    if constexpr (G >= 16) v += dpp_f32<0x140>(v);
    if constexpr (G >= 32)
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
    if constexpr (G >= 64)
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));
    return v;
}

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

// x prepared for the pairs of one word: for pair P, the low half is x[P] and
// the high half x[P + 8], each as bf16 hi + bf16 lo (x = hi + lo to 2^-16).
struct XPairs {
    uint32_t hi[8], lo[8];
};

// x = hi + lo exactly with hi = x truncated to bf16 (the top 16 bits); lo is
// then rounded to bf16 (round to nearest even), so hi + bf16(lo) matches x to
// a relative 2^-16. One perm packs the two hi halves of a pair.
__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
    const uint32_t ab = __float_as_uint(a), bb = __float_as_uint(b);
    hi = __builtin_amdgcn_perm(bb, ab, 0x07060302u);   // {a.hi16, b.hi16}
    const float ar = a - __uint_as_float(ab & 0xFFFF0000u);
    const float br = b - __uint_as_float(bb & 0xFFFF0000u);
    lo = f32_to_bf16_rne(ar) | (f32_to_bf16_rne(br) << 16);
}

__device__ __forceinline__ float ternary_word_dot(uint32_t w, const XPairs& xp, float acc) {
    float a0 = acc, a1 = 0.f;
#define E2M1_TPAIR(P)                                         \
    {                                                         \
        const uint32_t wp = ternary_pair<P>(w);               \
        a0 = dot2_bf16(wp, xp.hi[P], a0);                     \
        a1 = dot2_bf16(wp, xp.lo[P], a1);                     \
    }
    E2M1_TPAIR(0) E2M1_TPAIR(1) E2M1_TPAIR(2) E2M1_TPAIR(3)
    E2M1_TPAIR(4) E2M1_TPAIR(5) E2M1_TPAIR(6) E2M1_TPAIR(7)
#undef E2M1_TPAIR
    return a0 + a1;
}

// Fast path: K % 64 == 0, packed and x 16-byte aligned, K <= 4096. A group of
// G lanes covers one row (64 / G rows per wave, 16 waves per workgroup); lane
// gl owns the 64-column chunk gl. Per workgroup and pass: every thread first
// requests its x values for the split and its 16-byte weight chunk, then
// splits its share of x into bf16 hi/lo pairs in LDS; after one barrier each
// lane reads the pairs of its chunk and sums its row.
constexpr int kTernaryWaves = 16;
constexpr int kPairPitch = 68;   // dwords per chunk in LDS: 64 pair words + 4 (spreads the banks)

template <int G>
__global__ __launch_bounds__(kWave * kTernaryWaves) void ternary_kernel(const uint32_t* __restrict__ packed,
                                                                        const float* __restrict__ row_scale,
                                                                        const float* __restrict__ x,
                                                                        float* __restrict__ y, int n, int kq) {
    constexpr int kRowsPerWave = kWave / G;
    constexpr int kRowsPerBlock = kTernaryWaves * kRowsPerWave;
    __shared__ __attribute__((aligned(16))) uint32_t pairs[64 * kPairPitch];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int gl = lane & (G - 1);
    const int c = min(gl, kq - 1);
    const bool cvalid = gl < kq;
    const int npairs = kq * 32;   // (x[16 w + p], x[16 w + p + 8]) for p < 8, four words per chunk
    const uint4* pk = reinterpret_cast<const uint4*>(packed);

    for (int row0 = blockIdx.x * kRowsPerBlock; row0 < n; row0 += gridDim.x * kRowsPerBlock) {
        // x values of this thread's pairs, then its weight chunk (vector loads complete in order)
        float xa[2], xb[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int t = min((int)threadIdx.x + j * kWave * kTernaryWaves, npairs - 1);
            const int base = 64 * (t >> 5) + 16 * ((t >> 3) & 3) + (t & 7);
            xa[j] = x[base];
            xb[j] = x[base + 8];
        }
        const int row = row0 + wave * kRowsPerWave + lane / G;
        const uint4 w = load_nt16(pk + (int64_t)min(row, n - 1) * kq + c);
        const float s = row_scale[min(row, n - 1)];
        __syncthreads();   // the previous pass is done reading the pairs
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int t = (int)threadIdx.x + j * kWave * kTernaryWaves;
            if (t < npairs) {
                uint32_t hi, lo;
                split_pair(xa[j], xb[j], hi, lo);
                const int at = (t >> 5) * kPairPitch + 16 * ((t >> 3) & 3) + (t & 7);
                pairs[at] = hi;
                pairs[at + 8] = lo;
            }
        }
        __syncthreads();
        XPairs xp[4];
        {
            const uint4* pp = reinterpret_cast<const uint4*>(pairs + c * kPairPitch);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint4 h0 = pp[4 * q + 0], h1 = pp[4 * q + 1], l0 = pp[4 * q + 2], l1 = pp[4 * q + 3];
                xp[q].hi[0] = h0.x; xp[q].hi[1] = h0.y; xp[q].hi[2] = h0.z; xp[q].hi[3] = h0.w;
                xp[q].hi[4] = h1.x; xp[q].hi[5] = h1.y; xp[q].hi[6] = h1.z; xp[q].hi[7] = h1.w;
                xp[q].lo[0] = l0.x; xp[q].lo[1] = l0.y; xp[q].lo[2] = l0.z; xp[q].lo[3] = l0.w;
                xp[q].lo[4] = l1.x; xp[q].lo[5] = l1.y; xp[q].lo[6] = l1.z; xp[q].lo[7] = l1.w;
            }
        }
        const uint4 wv = cvalid ? w : make_uint4(0u, 0u, 0u, 0u);
        float acc = ternary_word_dot(wv.x, xp[0], 0.f);
        acc = ternary_word_dot(wv.y, xp[1], acc);
        acc = ternary_word_dot(wv.z, xp[2], acc);
        acc = ternary_word_dot(wv.w, xp[3], acc);
        acc = group_total<G>(acc);
        if (gl == G - 1 && row < n) y[row] = s * (2.0f * acc);
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

template <int G>
hipError_t run_fast(const uint32_t* packed, const float* s, const float* x, float* y, int n, int kq,
                    hipStream_t stream) {
    constexpr int kRowsPerBlock = kTernaryWaves * (kWave / G);
    // every row group its own workgroup up to four per compute unit, then passes
    const int want = (n + kRowsPerBlock - 1) / kRowsPerBlock;
    const int grid = min(want, 4 * device_cu_count());
    ternary_kernel<G><<<grid, kWave * kTernaryWaves, 0, stream>>>(packed, s, x, y, n, kq);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ternary(const uint32_t* packed, const float* row_scale, const float* x, float* y,
                          int64_t n, int64_t k, hipStream_t stream) {
    const int nn = (int)n;
    const bool aligned = (reinterpret_cast<uintptr_t>(packed) & 15u) == 0 &&
                         (reinterpret_cast<uintptr_t>(x) & 15u) == 0 && k % 64 == 0;
    if (aligned && k <= 64 * 64) {
        const int kq = (int)(k / 64);
        if (kq <= 8) return run_fast<8>(packed, row_scale, x, y, nn, kq, stream);
        if (kq <= 16) return run_fast<16>(packed, row_scale, x, y, nn, kq, stream);
        if (kq <= 32) return run_fast<32>(packed, row_scale, x, y, nn, kq, stream);
        return run_fast<64>(packed, row_scale, x, y, nn, kq, stream);
    }
    const int want = (nn + kWavesPerBlock - 1) / kWavesPerBlock;
    static int cap = 0;
    if (cap == 0) cap = resident_blocks(ternary_generic_kernel, 0);
    const int grid = want < cap ? want : cap;
    ternary_generic_kernel<<<grid, kThreads, 0, stream>>>(packed, row_scale, x, y, nn, (int)(k / 16));
    return hipGetLastError();
}

}  // namespace e2m1
