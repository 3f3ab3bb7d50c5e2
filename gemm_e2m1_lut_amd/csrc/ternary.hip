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
// chunk of K (one 16-byte load of four words) with its x pairs in registers;
// lanes cover a row in groups (64 lanes for K = 4096, fewer for short rows),
// the row total comes from a DPP-only reduction and is multiplied by the row
// scale once. Inputs the fast kernel cannot take (K % 64 != 0, K > 4096,
// unaligned pointers) use a one-wave-per-row kernel that adds, subtracts or
// skips each x directly.
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

// Weight pairs for v_dot2_f32_bf16. Fields p and p + 8 of a word (bits 2p,
// 2p+1 and 2p+16, 2p+17) are rotated to bits 8-9 and 24-25 and masked; the
// result is a v_perm_b32 selector that picks, from a 4-byte pool, the high
// byte of bf16 -0.5 (field 01), +0.5 (field 10) or 0 (fields 00 and 11), and
// 0x00 for the low bytes (selector byte 0 -> pool byte 0 = 0x00). One rotate,
// one mask and one perm give two weights as a bf16 pair of +/-0.5 or 0; the
// factor 2 is applied exactly with the row scale.
constexpr uint32_t kHalfPool = 0x003FBF00u;   // pool bytes: 00, BF (-0.5), 3F (+0.5), 00

template <int P>
__device__ __forceinline__ uint32_t ternary_pair(uint32_t w) {
    constexpr int kRotl = 8 - 2 * P;                     // bring bits 2P.. to bit 8
    const uint32_t r = kRotl == 0 ? w : __builtin_amdgcn_alignbit(w, w, (32 - kRotl) & 31);
    return __builtin_amdgcn_perm(0u, kHalfPool, r & 0x03000300u);
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

// Fast path: K % 64 == 0, packed and x 16-byte aligned, K <= 64 * G. A group
// of G lanes covers one row; lane gl owns the 64-column chunk gl (one 16-byte
// load of 4 words) for every row, with its x pairs in registers. R rows per
// group and pass; all loads unconditional (clamped, masked at use).
template <int G, int R>
__global__ __launch_bounds__(kThreads) void ternary_kernel(const uint32_t* __restrict__ packed,
                                                           const float* __restrict__ row_scale,
                                                           const float* __restrict__ x,
                                                           float* __restrict__ y, int n, int kq) {
    constexpr int kGroupsPerWave = kWave / G;
    const int lane = threadIdx.x & (kWave - 1);
    const int gl = lane & (G - 1);
    const int grp = lane / G;
    const int wave = blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    const int units = gridDim.x * kWavesPerBlock * kGroupsPerWave;
    const int unit = wave * kGroupsPerWave + grp;
    const int c = min(gl, kq - 1);
    const bool cvalid = gl < kq;

    XPairs xp[4];
    {
        const float4* xv = reinterpret_cast<const float4*>(x) + c * 16;
        float xs[64];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const float4 v = xv[q];
            xs[4 * q + 0] = v.x;
            xs[4 * q + 1] = v.y;
            xs[4 * q + 2] = v.z;
            xs[4 * q + 3] = v.w;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int p = 0; p < 8; ++p) split_pair(xs[16 * q + p], xs[16 * q + p + 8], xp[q].hi[p], xp[q].lo[p]);
    }
    const uint4* pk = reinterpret_cast<const uint4*>(packed);
    for (int pass = 0; (pass * units + wave * kGroupsPerWave) * R < n; ++pass) {
        const int row0 = (pass * units + unit) * R;
        uint4 w[R];
#pragma unroll
        for (int r = 0; r < R; ++r) w[r] = load_nt16(pk + (int64_t)min(row0 + r, n - 1) * kq + c);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint4 wv = cvalid ? w[r] : make_uint4(0u, 0u, 0u, 0u);
            float acc = ternary_word_dot(wv.x, xp[0], 0.f);
            acc = ternary_word_dot(wv.y, xp[1], acc);
            acc = ternary_word_dot(wv.z, xp[2], acc);
            acc = ternary_word_dot(wv.w, xp[3], acc);
            acc = group_total<G>(acc);
            const int row = row0 + r;
            if (gl == G - 1 && row < n) y[row] = row_scale[row] * (2.0f * acc);
        }
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

template <int G, int R>
hipError_t run_fast_r(const uint32_t* packed, const float* s, const float* x, float* y, int n,
                      int kq, int cap, hipStream_t stream) {
    const int rows_per_block = kWavesPerBlock * (kWave / G) * R;
    const int want = (n + rows_per_block - 1) / rows_per_block;
    const int grid = want < cap ? want : cap;
    ternary_kernel<G, R><<<grid, kThreads, 0, stream>>>(packed, s, x, y, n, kq);
    return hipGetLastError();
}

// Rows per group and pass: each group splits its x slice once (about as many
// VALU operations as two rows of weights), so a group takes 4 rows while that
// still leaves at least one wave per SIMD on every compute unit, else fewer.
template <int G>
hipError_t run_fast(const uint32_t* packed, const float* s, const float* x, float* y, int n, int kq,
                    hipStream_t stream) {
    static int cap1 = 0, cap2 = 0, cap4 = 0;
    if (cap1 == 0) {
        cap1 = resident_blocks(ternary_kernel<G, 1>, 0);
        cap2 = resident_blocks(ternary_kernel<G, 2>, 0);
        cap4 = resident_blocks(ternary_kernel<G, 4>, 0);
    }
    const int64_t groups_per_block = kWavesPerBlock * (kWave / G);
    const int64_t min_blocks = device_cu_count();   // one block (4 waves) per compute unit
    if ((n + 4 * groups_per_block - 1) / (4 * groups_per_block) >= min_blocks)
        return run_fast_r<G, 4>(packed, s, x, y, n, kq, cap4, stream);
    if ((n + 2 * groups_per_block - 1) / (2 * groups_per_block) >= min_blocks || cap1 * groups_per_block < n)
        return run_fast_r<G, 2>(packed, s, x, y, n, kq, cap2, stream);
    return run_fast_r<G, 1>(packed, s, x, y, n, kq, cap1, stream);
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
