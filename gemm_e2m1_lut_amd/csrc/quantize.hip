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
// half a byte written). MXFP4: two lanes per 32-column block, 16 elements per
// lane from two 16-byte loads; the block maximum is one DPP exchange with the
// partner lane; scaling by 2^(127 - e) is exact; rounding to nearest even is
// integer arithmetic on the fp32 pattern (one mantissa bit kept above 1,
// rint(2 a) below). NVFP4: one lane per 16-column block. Each lane stores its
// 16 codes as one 8-byte word; the block scale byte is stored by one lane.
#include "device.hpp"
#include "kernels.hpp"

namespace e2m1 {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// E2M1 code (sign in bit 3) of the value nearest to v, ties to the even code,
// |v| above 6 saturating to 6.
__device__ __forceinline__ uint32_t e2m1_rne(float v) {
    const uint32_t sign = (__float_as_uint(v) >> 28) & 8u;
    const float a = fabsf(v);
    uint32_t code;
    if (a < 1.0f) {
        code = (uint32_t)rintf(2.0f * a);   // 0, 0.5 or 1.0 -> codes 0, 1, 2
    } else {
        uint32_t b = __float_as_uint(a);
        b = (b + 0x1FFFFFu + ((b >> 22) & 1u)) & 0xFFC00000u;   // keep one mantissa bit, ties to even
        const uint32_t E = (b >> 23) - 127u;
        code = E >= 3u ? 7u : 2u + 2u * E + ((b >> 22) & 1u);
    }
    return sign | code;
}

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

// 16 codes (4 bits each, element 2i in the low nibble of byte i) of 16 values.
__device__ __forceinline__ uint2 pack16(const uint32_t (&c)[16]) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        lo |= c[i] << (4 * i);
        hi |= c[8 + i] << (4 * i);
    }
    return make_uint2(lo, hi);
}

__device__ __forceinline__ void load16(const uint16_t* p, float (&v)[16]) {
    const uint4 a = load_nt16(p), b = load_nt16(p + 8);
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[2 * i] = bf16_lo(w[i]);
        v[2 * i + 1] = bf16_hi(w[i]);
    }
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
    float v[16];
    load16(x + blk * 32 + half * 16, v);
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
    m = fmaxf(m, dpp_f32<0xB1>(m));   // the partner lane's half of the block
    const int e = m > 0.0f ? min(max(__builtin_amdgcn_frexp_expf(m) - 3 + 127, 0), 254) : 0;
    uint32_t c[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) c[i] = e2m1_rne(ldexpf(v[i], 127 - e));
    if (block < nblocks) {
        *reinterpret_cast<uint2*>(packed + block * 16 + half * 8) = pack16(c);
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
    float v[16];
    load16(x + block * 16, v);
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
    const uint32_t bs = e4m3_rne(m / (6.0f * g));
    const float eff = e4m3_to_f32(bs) * g;
    uint32_t c[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        c[i] = eff == 0.0f ? ((__float_as_uint(v[i]) >> 28) & 8u) : e2m1_rne(v[i] / eff);
    *reinterpret_cast<uint2*>(packed + block * 8) = pack16(c);
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
