// ternary_int8.hpp -- ternary weights and fp32 activations on the int8 matrix
// cores (v_mfma_i32_16x16x64_i8), shared by the widely-linear layer and the
// small-batch ternary GEMM.
//
// Ternary packing: FairyFuse blog post, section "三元 GEMV 的乘法消除原理"
// (16 weights per word, bit 2j+1 = +1, bit 2j = -1, neither = 0).
//
// Weights: one mask of a shifted word gives the fields j, j + 4, j + 8,
// j + 12 as v_perm_b32 selectors into a 4-byte pool, so one perm decodes four
// weights to int8 (11 VALU operations per 16-weight word). In the resulting
// A operand of word q, byte b of dword j is the weight of column
// 16 q + j + 4 b.
//
// Activations: one exponent S per group of values sharing a scale (from
// their largest |x|), so that |x 2^S| < 2^30; x 2^S = H + L 2^-30 with H its
// integer part and L = rint of its fraction times 2^30, both written as four
// signed base-256 digits. That is a 60-bit fixed point: every element of at
// least 2^-36 times the group's largest |x| is represented exactly, any other
// to within 2^-60 times that largest. Digit columns of the B operand list, for the same
// columns and in the same order as the A operand, digit i of H (worth
// 2^(8 i - S)) or of L (worth 2^(8 i - S - 30)); the int32 products are
// exact.
#pragma once

#include <type_traits>

#include "device.hpp"

namespace e2m1 {

typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void issue_fence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Largest value over the wave (DPP only), returned uniform.
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_f32<0xB1>(v));
    v = fmaxf(v, dpp_f32<0x4E>(v));
    v = fmaxf(v, dpp_f32<0x141>(v));
    v = fmaxf(v, dpp_f32<0x140>(v));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false)));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Exponent S with |x 2^S| < 2^30 for every |x| <= m (m = 0 gives 30).
__device__ __forceinline__ int slice_exponent(float m) {
    return 30 - __builtin_amdgcn_frexp_expf(m);
}

// The four signed base-256 digits of an integer |X| <= 2^30 as the bytes of
// one word: X + 0x808080 has unsigned low bytes u_i with X = sum (u_i - 128)
// 256^i + u_3 256^3, and xor 0x80 turns u_i into the int8 pattern of u_i - 128.
__device__ __forceinline__ uint32_t digit_bytes(int X) {
    return ((uint32_t)X + 0x00808080u) ^ 0x00808080u;
}

// Digits of x 2^S (|x 2^S| < 2^30): hi those of the integer part H, lo those
// of L = rint(fraction 2^30). t, its integer part and the fraction are exact
// in fp32 (scaling by a power of two, truncation, and the difference of a
// number and its integer part); only L rounds, for elements with bits below
// 2^(-S-30).
__device__ __forceinline__ void digits8(float x, int S, uint32_t& hi, uint32_t& lo) {
    const float t = ldexpf(x, S);
    const float h = truncf(t);
    hi = digit_bytes((int)h);
    lo = digit_bytes((int)rintf(ldexpf(t - h, 30)));
}

// 4 x 4 byte transpose: byte b of out[i] = byte i of in[b].
__device__ __forceinline__ void transpose4(const uint32_t (&in)[4], uint32_t (&out)[4]) {
    const uint32_t lo01 = __builtin_amdgcn_perm(in[1], in[0], 0x05010400u);
    const uint32_t hi01 = __builtin_amdgcn_perm(in[1], in[0], 0x07030602u);
    const uint32_t lo23 = __builtin_amdgcn_perm(in[3], in[2], 0x05010400u);
    const uint32_t hi23 = __builtin_amdgcn_perm(in[3], in[2], 0x07030602u);
    out[0] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
    out[1] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
    out[2] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
    out[3] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
}

// Ternary fields j, j + 4, j + 8, j + 12 of a word as int8 bytes 0..3: the
// masked field is a v_perm_b32 selector into the pool 00 (0), FF (-1 for
// field 01), 01 (+1 for field 10), 00 (field 11, not a valid weight: 0).
constexpr uint32_t kI8Pool = 0x0001FF00u;

template <int J>
__device__ __forceinline__ uint32_t ternary_quad(uint32_t w) {
    const uint32_t sel = (J == 0 ? w : (w >> (2 * J))) & 0x03030303u;
    return __builtin_amdgcn_perm(0u, kI8Pool, sel);
}

__device__ __forceinline__ i32x4 decode_word(uint32_t w) {
    i32x4 a;
    a.x = (int)ternary_quad<0>(w);
    a.y = (int)ternary_quad<1>(w);
    a.z = (int)ternary_quad<2>(w);
    a.w = (int)ternary_quad<3>(w);
    return a;
}

// Largest value over each 16-lane row (DPP only), in every lane of the row.
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_f32<0xB1>(v));
    v = fmaxf(v, dpp_f32<0x4E>(v));
    v = fmaxf(v, dpp_f32<0x141>(v));
    v = fmaxf(v, dpp_f32<0x140>(v));
    return v;
}

// Totals over the eight lanes that differ in lane bits 0..2 (the eight digit columns of an
// activation row), transposed: three pairings (row_half_mirror across bit 2, then quad_perm across
// bits 1 and 0) each halve the values a lane keeps, the lane whose bit is set keeping the upper
// half. On return v[0 .. M/8) of lane L hold the totals of value indices (L & 7) (M/8) + m.
template <int M>
__device__ __forceinline__ void digit_lane_totals(float (&v)[M], int lane) {
    static_assert(M % 8 == 0, "eight lanes, M / 8 values each");
    auto step = [&](auto ctrl, int bit, int h) {
        const bool upper = (lane >> bit) & 1;
#pragma unroll
        for (int j = 0; j < h; ++j) {
            const float keep = upper ? v[j + h] : v[j];
            const float send = upper ? v[j] : v[j + h];
            v[j] = keep + dpp_f32<decltype(ctrl)::value>(send);
        }
    };
    step(std::integral_constant<int, 0x141>{}, 2, M / 2);   // row_half_mirror: lane i <-> 7 - i
    step(std::integral_constant<int, 0x4E>{}, 1, M / 4);    // quad_perm [2,3,0,1]
    step(std::integral_constant<int, 0xB1>{}, 0, M / 8);    // quad_perm [1,0,3,2]
}

__device__ __forceinline__ i32x4 mfma_i8(i32x4 a, i32x4 b, i32x4 c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

}  // namespace e2m1
