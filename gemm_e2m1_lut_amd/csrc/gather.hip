// gather.hip -- NVFP4 embedding gather + dequantise (nvfp4_embedding_gather).
//
// Method: SGLang pull request 34222 digest, sections "实现拆解" (item 2) and
// "关键源码片段" (embedding()): gather the packed row and its E4M3 block
// scales for each token id, split every byte into the even (low nibble) and
// odd (high nibble) channel, look up the E2M1 magnitude and apply the sign
// bit, multiply by eff = float(block_scale) * float(global_scale) computed in
// fp32, and cast the fp32 product to bf16 (round to nearest even).
//
// gfx950 design. Pure data movement: 0.5625 bytes read per 2 written per
// channel, so the kernel is HBM-write bound. A thread owns one packed word (8
// channels) and writes their 16 bytes of bf16; the lanes of a wave cover
// consecutive words of a token row, so every store instruction writes one
// contiguous kilobyte. v_cvt_scalef32_pk_f32_fp4 with scale 1.0 yields the two
// signed E2M1 values of a byte exactly (code 8 is -0.0), the multiply is one
// IEEE fp32 multiply, and the bf16 rounding is v_cvt_pk_bf16_f32 (the integer
// round-half-even of device.hpp where a NaN can occur).
#include "device.hpp"
#include "kernels.hpp"

namespace e2m1 {
namespace {

constexpr int kThreads = 256;

// Two fp32 products -> two bf16, round to nearest even. v_cvt_pk_bf16_f32
// rounds exactly as f32_to_bf16_rne for every non-NaN input (subnormals and
// overflow to infinity included; checked on the device over 5 million
// patterns) but keeps a NaN's sign and payload, so it is used only when no
// product can be NaN.
__device__ __forceinline__ uint32_t bf16x2_rne(f32x2 v) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// One 32-bit code word (eight channels) -> four words of two bf16 each. The
// codes are finite, so the products are NaN only for a non-finite eff (an
// E4M3 NaN byte or a non-finite global scale); then every NaN is written as
// 0x7FC0.
__device__ __forceinline__ void dequant_word(uint32_t w, float eff, uint32_t* out) {
    const f32x2 v0 = fp4x2_to_f32x2<0>(w, 1.0f) * eff;
    const f32x2 v1 = fp4x2_to_f32x2<1>(w, 1.0f) * eff;
    const f32x2 v2 = fp4x2_to_f32x2<2>(w, 1.0f) * eff;
    const f32x2 v3 = fp4x2_to_f32x2<3>(w, 1.0f) * eff;
    if (__builtin_isfinite(eff)) {
        out[0] = bf16x2_rne(v0);
        out[1] = bf16x2_rne(v1);
        out[2] = bf16x2_rne(v2);
        out[3] = bf16x2_rne(v3);
    } else {
        out[0] = pack_bf16x2(v0.x, v0.y);
        out[1] = pack_bf16x2(v1.x, v1.y);
        out[2] = pack_bf16x2(v2.x, v2.y);
        out[3] = pack_bf16x2(v3.x, v3.y);
    }
}

// One thread per packed word (8 channels, half of a 16-channel scale group)
// and token row, kRows rows per thread: a 4-byte load, the group's E4M3 byte
// and one 16-byte store per row. A block covers kRows groups of
// `rows_per_block` token rows with `tpr` threads each (tpr a power of two) or,
// for long rows, a row segment of `tpr` words in each of `blocks_per_row`
// consecutive blocks. Consecutive lanes read consecutive words of a row and
// write one contiguous kilobyte per wave-wide store. Every id, code word and
// scale of a thread's rows is requested (indices clamped into range) before
// any of them is used, so the dependent id -> row loads of different rows
// overlap. Sixteen rows per thread put the whole 8192-id workload in flight in
// one round of workgroups (four rows per thread took two: 22.8-23.1 against
// 21.7 us for 8192 rows of 4096 channels).
constexpr int kRows = 16;

__global__ __launch_bounds__(kThreads) void gather_kernel(
    const uint32_t* __restrict__ table, const uint8_t* __restrict__ block_scale,
    const float* __restrict__ global_scale, const int64_t* __restrict__ ids,
    uint4* __restrict__ out, int64_t vocab, int64_t wpr, int64_t ntok,
    int32_t* __restrict__ err_flag, int tpr_log2, int64_t blocks_per_row) {
    const float g = *global_scale;
    const int tpr = 1 << tpr_log2;
    const int rows_per_block = kThreads >> tpr_log2;
    const int sub = threadIdx.x & (tpr - 1);
    const int64_t rows_per_iter = (int64_t)rows_per_block * kRows;
    const int64_t groups = (ntok + rows_per_iter - 1) / rows_per_iter;
    for (int64_t b = blockIdx.x; b < groups * blocks_per_row; b += gridDim.x) {
        const int64_t rg = b / blocks_per_row;
        const int64_t part = b - rg * blocks_per_row;
        const int64_t c = part * tpr + sub;
        const int64_t cc = c < wpr ? c : wpr - 1;
        int64_t t[kRows], id[kRows];
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
            t[i] = rg * rows_per_iter + (int64_t)i * rows_per_block + (threadIdx.x >> tpr_log2);
            id[i] = ids[t[i] < ntok ? t[i] : ntok - 1];
        }
        uint32_t p[kRows];
        uint32_t sb[kRows];
        if (vocab > 0) {   // an empty table is never read (it may be NULL): every row is out of range
#pragma unroll
            for (int i = 0; i < kRows; ++i) {
                const int64_t r = (id[i] >= 0 && id[i] < vocab) ? id[i] : 0;
                p[i] = __builtin_nontemporal_load(table + r * wpr + cc);
                sb[i] = block_scale[r * (wpr / 2) + (cc >> 1)];
            }
        } else {
#pragma unroll
            for (int i = 0; i < kRows; ++i) p[i] = sb[i] = 0u;
        }
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
            if (t[i] >= ntok || c >= wpr) continue;
            uint4* o = out + t[i] * wpr + c;
            if (id[i] < 0 || id[i] >= vocab) {
                *o = make_uint4(0u, 0u, 0u, 0u);
                if (err_flag != nullptr) *err_flag = 1;
                continue;
            }
            uint32_t w[4];
            dequant_word(p[i], e4m3_to_f32(sb[i]) * g, w);
            store_nt16(o, w[0], w[1], w[2], w[3]);
        }
    }
}

}  // namespace

hipError_t launch_nvfp4_gather(const uint8_t* table, const uint8_t* block_scale,
                               const float* global_scale, const int64_t* ids, uint16_t* out,
                               int64_t vocab, int64_t hidden, int64_t ntok, int32_t* err_flag,
                               hipStream_t stream) {
    const int64_t wpr = hidden / 8;   // packed words (and 16-byte output pieces) per row
    int tpr_log2 = 0;
    while ((1 << tpr_log2) < wpr && (1 << tpr_log2) < kThreads) ++tpr_log2;
    const int tpr = 1 << tpr_log2;
    const int64_t blocks_per_row = (wpr + tpr - 1) / tpr;
    const int rows_per_block = kThreads / tpr;
    const int64_t blocks = (ntok + (int64_t)rows_per_block * kRows - 1) / ((int64_t)rows_per_block * kRows) *
                           blocks_per_row;
    const int64_t cap = (int64_t)device_cu_count() * 64;
    const int grid = (int)(blocks < cap ? blocks : cap);
    gather_kernel<<<grid, kThreads, 0, stream>>>(reinterpret_cast<const uint32_t*>(table), block_scale,
                                                 global_scale, ids, reinterpret_cast<uint4*>(out),
                                                 vocab, wpr, ntok, err_flag, tpr_log2, blocks_per_row);
    return hipGetLastError();
}

}  // namespace e2m1
