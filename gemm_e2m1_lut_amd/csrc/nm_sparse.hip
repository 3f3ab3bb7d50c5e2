// nm_sparse.hip -- N:M structured-sparse weight times a few activation rows (nm_spmm).
//
// Format: sglang-jax wiki page on the N:M structured sparse matmul gap,
// sections "N:M 稀疏原理" and "3.1 Sparsifier": in every group of M
// consecutive columns of a weight row, N values are kept; their in-group
// positions are packed next_log2(M) bits each, 32 / bits per 32-bit word,
// entry i of the row at bit (i mod packing) * bits of word i / packing. Rows
// follow one another: values [rows, (k/M) N] bf16, positions [rows, words].
// Operation ("3.2": decompress the metadata and multiply): y[b][r] = sum over
// the kept entries of row r of value * x[b][column], fp32 accumulation.
//
// gfx950 design: instead of rebuilding a dense tile (the TPU kernel's route,
// which pays for the zeros), each kept value is multiplied by the activation
// at its column. A workgroup of four waves copies x (batch x K bf16) into LDS
// once and then walks rows, one wave per row; each lane takes eight
// consecutive kept values per 16-byte load (a wave reads 1 KB of contiguous
// values per instruction), reads the one or two metadata words holding their
// positions, and gathers x from LDS at group * M + position. With N and M
// fixed at compile time for the common configurations, the group and word
// arithmetic is shifts and multiplies by constants. Wave totals are DPP-only.
// Other configurations, activations too large for LDS, and unaligned rows
// take a kernel that reads x from memory, one entry per lane at a time.
#include "device.hpp"
#include "kernels.hpp"

namespace e2m1 {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxLdsElems = 32768;   // bf16 activations staged per workgroup (64 KB)

__host__ __device__ constexpr int nm_bits(int m) { return m <= 2 ? 1 : m <= 4 ? 2 : m <= 8 ? 3 : 4; }

template <bool kBf16Out>
__device__ __forceinline__ void nm_store(void* y, int64_t idx, float v) {
    if constexpr (kBf16Out)
        reinterpret_cast<uint16_t*>(y)[idx] = (uint16_t)f32_to_bf16_rne(v);
    else
        reinterpret_cast<float*>(y)[idx] = v;
}

template <int NN, int MM, int B, bool kBf16Out>
__global__ __launch_bounds__(kThreads) void nm_spmm_kernel(const uint16_t* __restrict__ values,
                                                           const uint32_t* __restrict__ meta,
                                                           const uint16_t* __restrict__ x, void* __restrict__ y,
                                                           int rows, int k) {
    constexpr int kBits = nm_bits(MM);
    constexpr int kPacking = 32 / kBits;
    constexpr uint32_t kPosMask = (1u << kBits) - 1u;
    extern __shared__ __attribute__((aligned(16))) uint16_t nm_x[];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int per_row = (k / MM) * NN;
    const int words = (per_row + kPacking - 1) / kPacking;

    // x -> LDS (B rows of k bf16, 16-byte chunks)
    for (int i = threadIdx.x; i < B * k / 8; i += kThreads)
        reinterpret_cast<uint4*>(nm_x)[i] = reinterpret_cast<const uint4*>(x)[i];
    __syncthreads();

    for (int row = blockIdx.x * kWaves + wave; row < rows; row += gridDim.x * kWaves) {   // wave-uniform
        const uint16_t* vrow = values + (size_t)row * per_row;
        const uint32_t* mrow = meta + (size_t)row * words;
        float acc[B];
#pragma unroll
        for (int b = 0; b < B; ++b) acc[b] = 0.f;
        for (int e0 = 8 * lane; e0 < per_row; e0 += 8 * kWave) {   // per_row % 8 == 0 on this path
            const uint4 v = load_nt16(vrow + e0);
            const int w0 = e0 / kPacking, w1 = min((e0 + 7) / kPacking, words - 1);
            const uint32_t m0 = mrow[w0], m1 = mrow[w1];
            const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int e = e0 + i;
                const int wi = e / kPacking;
                const uint32_t word = wi == w0 ? m0 : m1;
                const uint32_t pos = (word >> ((e - wi * kPacking) * kBits)) & kPosMask;
                const int col = (e / NN) * MM + (int)pos;
                const float wv = __uint_as_float((i & 1) ? (vv[i >> 1] & 0xFFFF0000u) : (vv[i >> 1] << 16));
#pragma unroll
                for (int b = 0; b < B; ++b)
                    acc[b] = fmaf(wv, __uint_as_float((uint32_t)nm_x[b * k + col] << 16), acc[b]);
            }
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const float s = group_sum<kWave>(acc[b]);
            if (lane == 0) nm_store<kBf16Out>(y, (int64_t)b * rows + row, s);
        }
    }
}

// Any N:M with M <= 16, any batch, x from memory: one wave per row, one entry per lane at a time.
template <bool kBf16Out>
__global__ __launch_bounds__(kThreads) void nm_spmm_generic_kernel(const uint16_t* __restrict__ values,
                                                                   const uint32_t* __restrict__ meta,
                                                                   const uint16_t* __restrict__ x,
                                                                   void* __restrict__ y, int batch, int rows,
                                                                   int k, int nn, int mm) {
    const int bits = nm_bits(mm), packing = 32 / bits;
    const uint32_t pmask = (1u << bits) - 1u;
    const int lane = threadIdx.x & (kWave - 1);
    const int per_row = (k / mm) * nn;
    const int words = (per_row + packing - 1) / packing;
    for (int row = blockIdx.x * kWaves + threadIdx.x / kWave; row < rows; row += gridDim.x * kWaves) {
        for (int b = 0; b < batch; ++b) {
            float acc = 0.f;
            for (int e = lane; e < per_row; e += kWave) {
                const uint32_t pos = (meta[(size_t)row * words + e / packing] >> ((e % packing) * bits)) & pmask;
                const int col = (e / nn) * mm + (int)min(pos, (uint32_t)mm - 1u);
                acc = fmaf(__uint_as_float((uint32_t)values[(size_t)row * per_row + e] << 16),
                           __uint_as_float((uint32_t)x[(size_t)b * k + col] << 16), acc);
            }
            acc = group_sum<kWave>(acc);
            if (lane == 0) nm_store<kBf16Out>(y, (int64_t)b * rows + row, acc);
        }
    }
}

template <int NN, int MM, int B, bool kBf16Out>
hipError_t run_nm(const uint16_t* values, const uint32_t* meta, const uint16_t* x, void* y, int rows, int k,
                  hipStream_t stream) {
    const size_t lds = (size_t)B * k * sizeof(uint16_t);
    static int per_cu = 0;
    if (per_cu == 0) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(nm_spmm_kernel<NN, MM, B, kBf16Out>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLdsElems * 2);
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, nm_spmm_kernel<NN, MM, B, kBf16Out>, kThreads,
                                                         lds) != hipSuccess ||
            per_cu < 1)
            per_cu = 1;
    }
    const int want = (rows + kWaves - 1) / kWaves;
    const int grid = min(want, per_cu * device_cu_count());
    nm_spmm_kernel<NN, MM, B, kBf16Out><<<grid, kThreads, lds, stream>>>(values, meta, x, y, rows, k);
    return hipGetLastError();
}

template <int NN, int MM, bool kBf16Out>
hipError_t dispatch_batch(int batch, const uint16_t* values, const uint32_t* meta, const uint16_t* x, void* y,
                          int rows, int k, hipStream_t stream) {
    switch (batch) {
        case 1: return run_nm<NN, MM, 1, kBf16Out>(values, meta, x, y, rows, k, stream);
        case 2: return run_nm<NN, MM, 2, kBf16Out>(values, meta, x, y, rows, k, stream);
        case 3: return run_nm<NN, MM, 3, kBf16Out>(values, meta, x, y, rows, k, stream);
        case 4: return run_nm<NN, MM, 4, kBf16Out>(values, meta, x, y, rows, k, stream);
        default: return hipErrorInvalidValue;   // the fast path takes batch <= 4 only
    }
}

template <bool kBf16Out>
hipError_t launch_nm_t(const uint16_t* values, const uint32_t* meta, const uint16_t* x, void* y, int batch,
                       int rows, int k, int nn, int mm, hipStream_t stream) {
    const int per_row = (k / mm) * nn;
    const bool fast = batch <= 4 && (int64_t)batch * k <= kMaxLdsElems && k % 8 == 0 && per_row % 8 == 0 &&
                      (reinterpret_cast<uintptr_t>(values) & 15u) == 0 && (reinterpret_cast<uintptr_t>(x) & 15u) == 0;
    if (fast) {
        if (nn == 2 && mm == 4) return dispatch_batch<2, 4, kBf16Out>(batch, values, meta, x, y, rows, k, stream);
        if (nn == 1 && mm == 4) return dispatch_batch<1, 4, kBf16Out>(batch, values, meta, x, y, rows, k, stream);
        if (nn == 4 && mm == 8) return dispatch_batch<4, 8, kBf16Out>(batch, values, meta, x, y, rows, k, stream);
        if (nn == 1 && mm == 2) return dispatch_batch<1, 2, kBf16Out>(batch, values, meta, x, y, rows, k, stream);
        if (nn == 8 && mm == 16) return dispatch_batch<8, 16, kBf16Out>(batch, values, meta, x, y, rows, k, stream);
    }
    const int want = (rows + kWaves - 1) / kWaves;
    const int grid = min(want, 8 * device_cu_count());
    nm_spmm_generic_kernel<kBf16Out><<<grid, kThreads, 0, stream>>>(values, meta, x, y, batch, rows, k, nn, mm);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_nm_spmm(const uint16_t* values, const uint32_t* meta, const uint16_t* x, void* y, bool out_bf16,
                          int64_t batch, int64_t rows, int64_t k, int nn, int mm, hipStream_t stream) {
    return out_bf16 ? launch_nm_t<true>(values, meta, x, y, (int)batch, (int)rows, (int)k, nn, mm, stream)
                    : launch_nm_t<false>(values, meta, x, y, (int)batch, (int)rows, (int)k, nn, mm, stream);
}

}  // namespace e2m1
