// device.hpp -- gfx950 device helpers shared by the kernels of libe2m1lut.so.
//
// Formats (the oracle keeps its own, independent copy of every table):
//   E2M1 code: bit 3 = sign, bits 0..2 index {0, 0.5, 1, 1.5, 2, 3, 4, 6}
//     (SGLang pull request 34222 digest, section "关键源码片段": the lookup
//     table of the NVFP4 embedding).
//   E8M0 block scale: one byte e per 32 columns, 2^(e-127) (vLLM pull request
//     51583 digest, section "功能与动机").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace e2m1 {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Word 3 of a buffer resource for raw 32-bit-addressed loads (gfx9 family): bounds-checked
// against the resource's byte count, zeros outside it.
constexpr int kBufferWord3 = 0x00020000;

// ------------------------------------------------- streaming loads / stores --
// Non-temporal (streaming) 16- and 8-byte accesses for data touched once.

__device__ __forceinline__ uint4 load_nt16(const void* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint2 load_nt8(const void* p) {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    return make_uint2(v.x, v.y);
}

__device__ __forceinline__ void store_nt16(void* p, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const u32x4 v = {a, b, c, d};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// ---------------------------------------------------------------- E8M0 ----

// Scale operand of the hardware FP4 conversions for an E8M0 byte. The
// conversions use only the exponent field of this fp32, with the E8M0 meaning
// (0 -> 2^-127, 255 -> NaN). The method keeps both zero codes at +0.0 for
// every exponent, 255 included (vLLM pull request 51583 digest, "实现拆解"
// item 4 and its zero-code test), so 255 is read as 254: zero codes then
// convert to zero, and non-zero codes are defined only for 2 <= e <= 252.
__device__ __forceinline__ float e8m0_scale(uint32_t e) {
    return __uint_as_float((e < 254u ? e : 254u) << 23);
}

// ------------------------------------------------- hardware FP4 -> bf16/f32 --
// v_cvt_scalef32_pk_{bf16,f32}_fp4 decode the two E2M1 codes of one byte of
// `word` (byte index = immediate) and multiply by `scale`. Element 0 of the
// result is the low nibble (the even column), element 1 the high nibble.

template <int kByte>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t word, float scale) {
    bf16x2 v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, kByte);
    return __builtin_bit_cast(uint32_t, v);
}

template <int kByte>
__device__ __forceinline__ f32x2 fp4x2_to_f32x2(uint32_t word, float scale) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, scale, kByte);
}

// acc + w.lo * x.lo + w.hi * x.hi with bf16 pairs packed in 32-bit words.
__device__ __forceinline__ float dot2_bf16(uint32_t w, uint32_t x, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                           __builtin_bit_cast(bf16x2, x), acc, false);
}

// ------------------------------------------------------------ reductions ----

template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, true));
}

// Sum over aligned groups of kLanes lanes (kLanes in {1,2,4,8,16,32,64});
// every lane of a group ends with the group total.
template <int kLanes>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (kLanes >= 2) v += dpp_f32<0xB1>(v);    // quad_perm [1,0,3,2]
    if constexpr (kLanes >= 4) v += dpp_f32<0x4E>(v);    // quad_perm [2,3,0,1]
    if constexpr (kLanes >= 8) v += dpp_f32<0x141>(v);   // row_half_mirror
    if constexpr (kLanes >= 16) v += dpp_f32<0x140>(v);  // row_mirror
    if constexpr (kLanes >= 32) v += __shfl_xor(v, 16, kWave);
    if constexpr (kLanes >= 64) v += __shfl_xor(v, 32, kWave);
    return v;
}

// ------------------------------------------------------------ bf16 / fp32 --

// bf16 pattern of a float, round to nearest, ties to even; NaN -> 0x7FC0.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// OCP E4M3 (e4m3fn) byte -> fp32: bias 7, subnormals at exponent 0, no
// infinities, S.1111.111 = NaN.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
    uint32_t s = (b & 0x80u) << 24;
    uint32_t e = (b >> 3) & 15u;
    uint32_t m = b & 7u;
    if (e == 15u && m == 7u) return __uint_as_float(0x7FC00000u);
    if (e == 0u) return __uint_as_float(__float_as_uint((float)m * 0x1p-9f) | s);
    return __uint_as_float(s | ((e + 120u) << 23) | (m << 20));
}

}  // namespace e2m1
