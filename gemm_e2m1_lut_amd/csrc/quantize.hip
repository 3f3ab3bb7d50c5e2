// quantize.hip -- MXFP4 and NVFP4 quantizers (mxfp4_quantize, nvfp4_quantize):
// the encode side of the formats the rest of the library decodes.
//
// The pages use quantized weights without printing an encoder: the MoE test
// of the vLLM pull request 51583 digest (section "关键源码片段") quantizes
// bf16 weights to MXFP4 codes [.., K/2] and E8M0 scales [.., K/32]; the
// SGLang pull request 34222 digest only dequantises NVFP4 (E2M1 times an E4M3
// block scale per 16 columns times an fp32 global scale). Rounding rule taken:
// an element is the E2M1 value nearest to its scaled input, ties to the code
// whose last bit is 0, magnitudes above 6 saturate to 6, the sign bit is the
// input's. MXFP4 block exponent: floor(log2(amax)) - 2 (the largest element
// lands in [4, 8)), biased by 127 and clamped to 0..254, 0 for an all-zero
// block. NVFP4 block scale: the E4M3 value nearest to fl32(amax / fl32(6 g)),
// saturating at 448; elements are encoded from fl32(x / eff) with
// eff = fl32(e4m3(bs) * g), the product the dequantisation forms.
//
// gfx950 design: both are streaming kernels (2 bytes read per element, about
// half a byte written). The E2M1 rounding is the hardware's:
// v_cvt_scalef32_pk_fp4_{bf16,f32} turn two values into two E2M1 codes,
// dividing by 2^E for the exponent field E of the scale operand and rounding
// to nearest with ties to the even code, saturating at 6 and keeping the sign
// of zero -- exactly the rule above (checked on the device against it for
// every finite bf16 pattern at scales 2^-127 .. 2^100 and for 1.3 million
// fp32 values, including every value within 300 ulps of each rounding
// boundary). MXFP4: two lanes per 32-column block, 16 elements per lane from
// two 16-byte loads; the block maximum is an integer maximum of the magnitude
// patterns (finite bf16 magnitudes order like their patterns) and one DPP
// exchange with the partner lane; its exponent field gives e, and the codes
// come straight from the bf16 pairs with scale 2^(e-127), eight conversions
// per lane. NVFP4: one lane per 16-column block; the codes of fl32(x / eff)
// come from a reciprocal multiply bracketed on both sides (IEEE divisions
// only near a rounding boundary), converted with scale 1. Each lane stores its 16 codes as
// one 8-byte word; the block scale byte is stored by one lane.
#include "device.hpp"
#include "kernels.hpp"

namespace e2m1 {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// E4M3 (e4m3fn) byte of the value nearest to t >= 0, ties to an even
// mantissa, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_rne(float t) {
    if (!(t < 448.0f)) return 0x7Eu;
    if (t < 0.015625f) return (uint32_t)rintf(t * 512.0f);   // subnormals m * 2^-9 (8 -> 2^-6 = byte 8)
    uint32_t b = __float_as_uint(t);
    b = (b + 0x7FFFFu + ((b >> 20) & 1u)) & 0xFFF00000u;      // keep three mantissa bits, ties to even
    const uint32_t code = (((b >> 23) - 120u) << 3) | ((b >> 20) & 7u);
    return code > 0x7Eu ? 0x7Eu : code;
}

// Eight bf16 pairs (16 elements) of one lane.
__device__ __forceinline__ void load16(const uint16_t* p, uint32_t (&w)[8]) {
    const uint4 a = load_nt16(p), b = load_nt16(p + 8);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
}

// Largest magnitude pattern of the 16 bf16 values (finite inputs).
__device__ __forceinline__ uint32_t amax_pattern(const uint32_t (&w)[8]) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t a = w[i] & 0x7FFF7FFFu;
        m = max(m, max(a & 0xFFFFu, a >> 16));
    }
    return m;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Byte `sel` of `old` replaced by the codes of a (low nibble) and b, scale 1.
__device__ __forceinline__ uint32_t cvt_fp4_sel(uint32_t old, float a, float b, int sel) {
    switch (sel) {   // the byte index is an immediate of the instruction
        case 0: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, 0);
        case 1: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, 1);
        case 2: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, 2);
        default: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, 3);
    }
}

// Codes of 16 bf16 values divided by 2^E (E the exponent field of sc):
// byte i of the result holds element 2 i (low nibble) and 2 i + 1.
__device__ __forceinline__ uint2 encode16_bf16(const uint32_t (&w)[8], float sc) {
    uint32_t lo = 0, hi = 0;
    lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(lo, __builtin_bit_cast(bf16x2_t, w[0]), sc, 0);
    lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(lo, __builtin_bit_cast(bf16x2_t, w[1]), sc, 1);
    lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(lo, __builtin_bit_cast(bf16x2_t, w[2]), sc, 2);
    lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(lo, __builtin_bit_cast(bf16x2_t, w[3]), sc, 3);
    hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(hi, __builtin_bit_cast(bf16x2_t, w[4]), sc, 0);
    hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(hi, __builtin_bit_cast(bf16x2_t, w[5]), sc, 1);
    hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(hi, __builtin_bit_cast(bf16x2_t, w[6]), sc, 2);
    hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(hi, __builtin_bit_cast(bf16x2_t, w[7]), sc, 3);
    return make_uint2(lo, hi);
}

// Lanes 2 j and 2 j + 1 own block j of the flattened input (every row is a
// whole number of blocks): 16 elements each.
__global__ __launch_bounds__(kThreads) void mxfp4_quantize_kernel(const uint16_t* __restrict__ x,
                                                                   uint8_t* __restrict__ packed,
                                                                   uint8_t* __restrict__ scales,
                                                                   int64_t nblocks) {
    const int64_t lane_id = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t block = lane_id >> 1;
    const int half = (int)(lane_id & 1);
    const int64_t blk = block < nblocks ? block : nblocks - 1;   // the last wave may run past the end
    uint32_t w[8];
    load16(x + blk * 32 + half * 16, w);
    uint32_t m = amax_pattern(w);
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, true));   // partner lane's half
    // floor(log2(amax)) - 2 + 127 is the exponent field minus 2 (subnormal and zero maxima give 0)
    const int e = max((int)(m >> 7) - 2, 0);
    const uint2 codes = encode16_bf16(w, __uint_as_float((uint32_t)e << 23));
    if (block < nblocks) {
        *reinterpret_cast<uint2*>(packed + block * 16 + half * 8) = codes;
        if (half == 0) scales[block] = (uint8_t)e;
    }
}

// Lane j owns block j (16 elements) of the flattened input.
__global__ __launch_bounds__(kThreads) void nvfp4_quantize_kernel(const uint16_t* __restrict__ x,
                                                                   const float* __restrict__ global_scale,
                                                                   uint8_t* __restrict__ packed,
                                                                   uint8_t* __restrict__ block_scale,
                                                                   int64_t nblocks) {
    const int64_t block = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (block >= nblocks) return;
    const float g = *global_scale;
    uint32_t w[8];
    load16(x + block * 16, w);
    const float m = __uint_as_float(amax_pattern(w) << 16);
    const uint32_t bs = e4m3_rne(m / (6.0f * g));
    const float eff = e4m3_to_f32(bs) * g;
    uint32_t lo = 0, hi = 0;
    if (eff == 0.0f) {   // signed zero codes
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t c = ((w[i] >> 12) & 8u) | ((w[i] >> 24) & 0x80u);   // sign of element 2 i, 2 i + 1
            if (i < 4) lo |= c << (8 * i);
            else hi |= c << (8 * (i - 4));
        }
    } else {
        // The code of fl32(x / eff) without the divisions where possible: with
        // q = x * rcp(eff) (v_rcp_f32 within one ulp), fl32(x / eff) lies within
        // 2^-22 of q relatively, and the E2M1 code is monotonic in q, so when
        // q (1 - 2^-18) and q (1 + 2^-18) get the same code, fl32(x / eff)
        // gets it too. A lane with any pair where they differ (q near a
        // rounding boundary), or with eff outside [2^-125, 2^125], divides.
        const float rinv = __builtin_amdgcn_rcpf(eff);
        uint32_t lo2 = 0, hi2 = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float q0 = bf16_lo(w[i]) * rinv, q1 = bf16_hi(w[i]) * rinv;
            const float d0 = q0 * 0x1.00001p-18f, d1 = q1 * 0x1.00001p-18f;
            if (i < 4) {
                lo = cvt_fp4_sel(lo, q0 - d0, q1 - d1, i);
                lo2 = cvt_fp4_sel(lo2, q0 + d0, q1 + d1, i);
            } else {
                hi = cvt_fp4_sel(hi, q0 - d0, q1 - d1, i - 4);
                hi2 = cvt_fp4_sel(hi2, q0 + d0, q1 + d1, i - 4);
            }
        }
        if (lo != lo2 || hi != hi2 || !(eff >= 0x1p-125f && eff <= 0x1p125f)) {
            lo = 0;
            hi = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float q0 = bf16_lo(w[i]) / eff, q1 = bf16_hi(w[i]) / eff;
                if (i < 4) lo = cvt_fp4_sel(lo, q0, q1, i);
                else hi = cvt_fp4_sel(hi, q0, q1, i - 4);
            }
        }
    }
    *reinterpret_cast<uint2*>(packed + block * 8) = make_uint2(lo, hi);
    block_scale[block] = (uint8_t)bs;
}

}  // namespace

hipError_t launch_mxfp4_quantize(const uint16_t* x, uint8_t* packed, uint8_t* scales, int64_t nblocks,
                                 hipStream_t stream) {
    const int64_t lanes = 2 * nblocks;
    const int64_t grid = (lanes + kThreads - 1) / kThreads;
    mxfp4_quantize_kernel<<<(unsigned)grid, kThreads, 0, stream>>>(x, packed, scales, nblocks);
    return hipGetLastError();
}

hipError_t launch_nvfp4_quantize(const uint16_t* x, const float* global_scale, uint8_t* packed,
                                 uint8_t* block_scale, int64_t nblocks, hipStream_t stream) {
    const int64_t grid = (nblocks + kThreads - 1) / kThreads;
    nvfp4_quantize_kernel<<<(unsigned)grid, kThreads, 0, stream>>>(x, global_scale, packed, block_scale,
                                                                   nblocks);
    return hipGetLastError();
}

}  // namespace e2m1
