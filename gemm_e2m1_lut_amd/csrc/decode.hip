// decode.hip -- MXFP4 -> bf16 unpack (dequant_decode).
//
// Method: vLLM pull request 51583 digest, sections "功能与动机" and
// "关键源码片段" (vec.h): each 4-bit code is looked up in a bf16 table, the
// E8M0 block scale is applied as an integer add of (e-127)*2^7 to the 16-bit
// pattern, and lanes holding one of the two zero codes are written as +0.0.
//
// gfx950 design. One thread owns one packed word (8 codes of one 32-column
// scale block): a 4-byte load, the block's scale byte, 16 bytes of bf16 out,
// so each wave stores one contiguous kilobyte per instruction. Because the
// codes of a block share one addend, the thread adds it to the eight magnitude
// patterns once (packed 16-bit adds) instead of once per lane -- the same
// integer sum -- and keeps the zero magnitude at +0 (the zero forcing). The scaled table is then
// split into a low-byte plane and a high-byte plane of 8 bytes each, so one
// v_perm_b32 looks up four codes in one plane. The sign (bit 3 of the code) is
// XORed into the high byte for non-zero magnitudes: adding 0x8000 modulo 2^16
// is the same as flipping bit 15, so signed and unsigned codes share a table.
// Memory-bound: 16.5 bytes in, 64 bytes out per 32 codes (write-dominated).
#include "device.hpp"
#include "kernels.hpp"

namespace e2m1 {
namespace {

// bf16 patterns of the E2M1 magnitudes, two per word (even index in the low
// half): {0x0000, 0x3F00}, {0x3F80, 0x3FC0}, {0x4000, 0x4040}, {0x4080, 0x40C0}.
constexpr uint32_t kMag01 = 0x3F000000u;
constexpr uint32_t kMag23 = 0x3FC03F80u;
constexpr uint32_t kMag45 = 0x40404000u;
constexpr uint32_t kMag67 = 0x40C04080u;

// v_perm_b32 selectors: byte i of the result is byte sel_i of {src0:src1}
// (src1 supplies bytes 0..3, src0 bytes 4..7).
constexpr uint32_t kSelLoBytes = 0x06040200u;   // bytes 0,2 of src1 then of src0
constexpr uint32_t kSelHiBytes = 0x07050301u;   // bytes 1,3 of src1 then of src0
constexpr uint32_t kSelPairs01 = 0x05010400u;   // {lo.b0, hi.b0, lo.b1, hi.b1}
constexpr uint32_t kSelPairs23 = 0x07030602u;   // {lo.b2, hi.b2, lo.b3, hi.b3}
constexpr uint32_t kSelHalf0 = 0x05040100u;     // {src1.lo16, src0.lo16}
constexpr uint32_t kSelHalf1 = 0x07060302u;     // {src1.hi16, src0.hi16}
// 0x80 in each byte whose magnitude index (0..7) is non-zero.
constexpr uint32_t kNonZero03 = 0x80808000u;
constexpr uint32_t kNonZero47 = 0x80808080u;

struct BytePlanes {
    uint32_t lo03, lo47, hi03, hi47;
};

__device__ __forceinline__ uint32_t perm(uint32_t src0, uint32_t src1, uint32_t sel) {
    return __builtin_amdgcn_perm(src0, src1, sel);
}

__device__ __forceinline__ uint32_t add16x2(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, a) + __builtin_bit_cast(u16x2, b));
}

// Table of the eight magnitudes with the block's exponent addend applied.
__device__ __forceinline__ BytePlanes scaled_planes(uint32_t e8m0) {
    const uint32_t add = ((e8m0 - 127u) << 7) & 0xFFFFu;
    const uint32_t add2 = add | (add << 16);
    const uint32_t p01 = add16x2(kMag01, add2) & 0xFFFF0000u;   // magnitude 0 stays +0
    const uint32_t p23 = add16x2(kMag23, add2);
    const uint32_t p45 = add16x2(kMag45, add2);
    const uint32_t p67 = add16x2(kMag67, add2);
    BytePlanes t;
    t.lo03 = perm(p23, p01, kSelLoBytes);
    t.hi03 = perm(p23, p01, kSelHiBytes);
    t.lo47 = perm(p67, p45, kSelLoBytes);
    t.hi47 = perm(p67, p45, kSelHiBytes);
    return t;
}

// Eight codes (four bytes) -> four words of two bf16 each, columns in order.
__device__ __forceinline__ void decode_word(uint32_t p, const BytePlanes& t, uint32_t* out) {
    const uint32_t sel_even = p & 0x07070707u;          // magnitudes of the low nibbles
    const uint32_t sel_odd = (p >> 4) & 0x07070707u;    // magnitudes of the high nibbles
    const uint32_t lo_e = perm(t.lo47, t.lo03, sel_even);
    const uint32_t lo_o = perm(t.lo47, t.lo03, sel_odd);
    uint32_t hi_e = perm(t.hi47, t.hi03, sel_even);
    uint32_t hi_o = perm(t.hi47, t.hi03, sel_odd);
    hi_e ^= (p << 4) & perm(kNonZero47, kNonZero03, sel_even);   // sign bit 3 -> bit 7
    hi_o ^= p & perm(kNonZero47, kNonZero03, sel_odd);           // sign bit 7 already in place
    const uint32_t e01 = perm(hi_e, lo_e, kSelPairs01);
    const uint32_t e23 = perm(hi_e, lo_e, kSelPairs23);
    const uint32_t o01 = perm(hi_o, lo_o, kSelPairs01);
    const uint32_t o23 = perm(hi_o, lo_o, kSelPairs23);
    out[0] = perm(o01, e01, kSelHalf0);
    out[1] = perm(o01, e01, kSelHalf1);
    out[2] = perm(o23, e23, kSelHalf0);
    out[3] = perm(o23, e23, kSelHalf1);
}

constexpr int kThreads = 256;

// One lane per packed word (8 codes): a 4-byte load, the word's scale byte
// (shared by the 4 words of a 32-column block), one 16-byte store. A wave
// takes runs of 64 kWordsPerLane consecutive words, lane l the words
// 64 j + l: the loads of all kWordsPerLane words (and their scale bytes) are
// issued before any is decoded, and every store instruction writes one
// contiguous kilobyte. (One word per lane and iteration kept a single 4-byte
// load in flight per lane: 29.1 against 27.5 us for 14336 x 4096; four words
// per lane measured the same as eight, sixteen 29.1 us.)
constexpr int kWordsPerLane = 8;

__global__ __launch_bounds__(kThreads) void decode_kernel(const uint32_t* __restrict__ packed,
                                                          const uint8_t* __restrict__ scales,
                                                          uint4* __restrict__ out,
                                                          int64_t nwords) {
    const int lane = threadIdx.x & (kWave - 1);
    constexpr int64_t kRun = (int64_t)kWave * kWordsPerLane;   // words per wave and iteration
    const int64_t nruns = (nwords + kRun - 1) / kRun;
    const int64_t waves = (int64_t)gridDim.x * (kThreads / kWave);
    for (int64_t run = (int64_t)blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave; run < nruns;
         run += waves) {   // wave-uniform
        const int64_t base = run * kRun + lane;
        uint32_t p[kWordsPerLane];
        uint8_t e[kWordsPerLane];
#pragma unroll
        for (int j = 0; j < kWordsPerLane; ++j) {
            const int64_t i = min(base + (int64_t)kWave * j, nwords - 1);
            p[j] = __builtin_nontemporal_load(packed + i);
            e[j] = scales[i >> 2];
        }
#pragma unroll
        for (int j = 0; j < kWordsPerLane; ++j) {
            const int64_t i = base + (int64_t)kWave * j;
            if (i < nwords) {
                uint32_t w[4];
                decode_word(p[j], scaled_planes(e[j]), w);
                store_nt16(out + i, w[0], w[1], w[2], w[3]);
            }
        }
    }
}

__global__ __launch_bounds__(kThreads) void fill_zero_kernel(uint16_t* __restrict__ dst,
                                                             int64_t count) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < count; i += stride)
        dst[i] = 0u;
}

}  // namespace

hipError_t launch_decode(const uint8_t* packed, const uint8_t* scales, uint16_t* out,
                         int64_t nblocks, hipStream_t stream) {
    const int64_t nwords = nblocks * 4;
    const int64_t want = (nwords + (int64_t)kThreads * kWordsPerLane - 1) / ((int64_t)kThreads * kWordsPerLane);
    const int64_t cap = (int64_t)device_cu_count() * 32;
    const int grid = (int)(want < cap ? want : cap);
    decode_kernel<<<grid, kThreads, 0, stream>>>(reinterpret_cast<const uint32_t*>(packed), scales,
                                                 reinterpret_cast<uint4*>(out), nwords);
    return hipGetLastError();
}

hipError_t launch_fill_zero_u16(uint16_t* dst, int64_t count, hipStream_t stream) {
    if (count <= 0) return hipSuccess;
    const int64_t want = (count + kThreads - 1) / kThreads;
    const int grid = (int)(want < 4096 ? want : 4096);
    fill_zero_kernel<<<grid, kThreads, 0, stream>>>(dst, count);
    return hipGetLastError();
}

}  // namespace e2m1
