// gather.hip -- NVFP4 embedding gather + dequantise (nvfp4_embedding_gather).
//
// Method: SGLang pull request 34222 digest, sections "实现拆解" (item 2) and
// "关键源码片段" (embedding()): gather the packed row and its E4M3 block
// scales for each token id, split every byte into the even (low nibble) and
// odd (high nibble) channel, look up the E2M1 magnitude and apply the sign
// bit, multiply by eff = float(block_scale) * float(global_scale) computed in
// fp32, and cast the fp32 product to bf16 (round to nearest even).
//
// gfx950 design. Pure data movement: 2.25 bytes read per 4 written per pair
// of channels, so the kernel is HBM-write bound. A thread owns one 32-channel
// chunk (16 bytes of codes, two block scales, 64 bytes of output); groups of
// threads cover one token row so the id is read once per group and rows are
// gathered with full 16-byte loads and stores. v_cvt_scalef32_pk_f32_fp4 with
// scale 1.0 yields the two signed E2M1 values of a byte exactly (code 8 is
// -0.0), the multiply is one IEEE fp32 multiply, and the bf16 rounding is the
// integer round-half-even of device.hpp. Tables whose rows are not 16-byte
// aligned (hidden % 32 != 0) use 16-channel chunks with 8-byte loads.
#include "device.hpp"
#include "kernels.hpp"

namespace e2m1 {
namespace {

constexpr int kThreads = 256;

// One 32-bit code word (eight channels) -> four words of two bf16 each.
__device__ __forceinline__ void dequant_word(uint32_t w, float eff, uint32_t* out) {
    const f32x2 v0 = fp4x2_to_f32x2<0>(w, 1.0f);
    const f32x2 v1 = fp4x2_to_f32x2<1>(w, 1.0f);
    const f32x2 v2 = fp4x2_to_f32x2<2>(w, 1.0f);
    const f32x2 v3 = fp4x2_to_f32x2<3>(w, 1.0f);
    out[0] = pack_bf16x2(v0.x * eff, v0.y * eff);
    out[1] = pack_bf16x2(v1.x * eff, v1.y * eff);
    out[2] = pack_bf16x2(v2.x * eff, v2.y * eff);
    out[3] = pack_bf16x2(v3.x * eff, v3.y * eff);
}

// kChunk = channels per thread-chunk (32: 16-byte loads, 16: 8-byte loads).
template <int kChunk>
__global__ __launch_bounds__(kThreads) void gather_kernel(
    const uint8_t* __restrict__ table, const uint8_t* __restrict__ block_scale,
    const float* __restrict__ global_scale, const int64_t* __restrict__ ids,
    uint16_t* __restrict__ out, int64_t vocab, int64_t hidden, int64_t ntok,
    int32_t* __restrict__ err_flag, int threads_per_row) {
    const float g = *global_scale;
    const int64_t cpr = hidden / kChunk;                    // chunks per row
    const int rows_per_block = kThreads / threads_per_row;
    const int sub = threadIdx.x % threads_per_row;
    const int64_t row_stride = (int64_t)gridDim.x * rows_per_block;
    for (int64_t t = (int64_t)blockIdx.x * rows_per_block + threadIdx.x / threads_per_row; t < ntok;
         t += row_stride) {
        const int64_t id = ids[t];
        uint16_t* orow = out + t * hidden;
        if (id < 0 || id >= vocab) {
            for (int64_t c = sub; c < cpr; c += threads_per_row) {
                if constexpr (kChunk == 32) {
                    uint4* o = reinterpret_cast<uint4*>(orow + c * 32);
                    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
                    o[0] = z; o[1] = z; o[2] = z; o[3] = z;
                } else {
                    uint4* o = reinterpret_cast<uint4*>(orow + c * 16);
                    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
                    o[0] = z; o[1] = z;
                }
            }
            if (err_flag != nullptr && sub == 0) *err_flag = 1;
            continue;
        }
        const uint8_t* prow = table + id * (hidden / 2);
        const uint8_t* srow = block_scale + id * (hidden / 16);
        for (int64_t c = sub; c < cpr; c += threads_per_row) {
            uint32_t w[16];
            if constexpr (kChunk == 32) {
                const uint4 p = load_nt16(reinterpret_cast<const uint4*>(prow) + c);
                const float eff0 = e4m3_to_f32(srow[2 * c]) * g;
                const float eff1 = e4m3_to_f32(srow[2 * c + 1]) * g;
                dequant_word(p.x, eff0, w + 0);
                dequant_word(p.y, eff0, w + 4);
                dequant_word(p.z, eff1, w + 8);
                dequant_word(p.w, eff1, w + 12);
                uint4* o = reinterpret_cast<uint4*>(orow + c * 32);
                store_nt16(o + 0, w[0], w[1], w[2], w[3]);
                store_nt16(o + 1, w[4], w[5], w[6], w[7]);
                store_nt16(o + 2, w[8], w[9], w[10], w[11]);
                store_nt16(o + 3, w[12], w[13], w[14], w[15]);
            } else {
                const uint2 p = load_nt8(reinterpret_cast<const uint2*>(prow) + c);
                const float eff = e4m3_to_f32(srow[c]) * g;
                dequant_word(p.x, eff, w + 0);
                dequant_word(p.y, eff, w + 4);
                uint4* o = reinterpret_cast<uint4*>(orow + c * 16);
                store_nt16(o + 0, w[0], w[1], w[2], w[3]);
                store_nt16(o + 1, w[4], w[5], w[6], w[7]);
            }
        }
    }
}

}  // namespace

hipError_t launch_nvfp4_gather(const uint8_t* table, const uint8_t* block_scale,
                               const float* global_scale, const int64_t* ids, uint16_t* out,
                               int64_t vocab, int64_t hidden, int64_t ntok, int32_t* err_flag,
                               hipStream_t stream) {
    const bool wide = hidden % 32 == 0 && (reinterpret_cast<uintptr_t>(table) & 15u) == 0 &&
                      (reinterpret_cast<uintptr_t>(out) & 15u) == 0;
    const int chunk = wide ? 32 : 16;
    const int64_t cpr = hidden / chunk;
    int tpr = 1;
    while (tpr < cpr && tpr < kThreads) tpr *= 2;
    const int rows_per_block = kThreads / tpr;
    const int64_t want = (ntok + rows_per_block - 1) / rows_per_block;
    const int64_t cap = (int64_t)device_cu_count() * 16;
    const int grid = (int)(want < cap ? want : cap);
    if (wide)
        gather_kernel<32><<<grid, kThreads, 0, stream>>>(table, block_scale, global_scale, ids, out,
                                                         vocab, hidden, ntok, err_flag, tpr);
    else
        gather_kernel<16><<<grid, kThreads, 0, stream>>>(table, block_scale, global_scale, ids, out,
                                                         vocab, hidden, ntok, err_flag, tpr);
    return hipGetLastError();
}

}  // namespace e2m1
