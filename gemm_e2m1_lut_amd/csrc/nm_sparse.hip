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
// at its column. A workgroup of eight waves copies x into LDS once and then
// walks rows, one wave per row:
//   * each lane takes eight consecutive kept values per 16-byte load (a wave
//     reads 1 KB of contiguous values per instruction), two such chunks in
//     flight, and the one metadata word (two when 8 entries can straddle a
//     word, as with 3-bit positions) holding their positions;
//   * the eight entries of a lane cover one span of 8 M / N columns, so x is
//     staged span by span with 4 or 8 bytes of padding after each span: the
//     spans of neighbouring lanes then start in different LDS banks instead of
//     every eighth lane colliding;
//   * for one activation row x is staged as is and two entries' activations
//     are read as 2-byte loads packed into one bf16 pair; for 2..4 rows x is
//     staged interleaved, [column][row] (2 or 4 slots per column), so one 4-
//     or 8-byte LDS read per entry serves every row;
//   * products are v_dot2_f32_bf16 on (value pair, activation pair), fp32
//     accumulation, wave totals DPP-only.
// With N and M fixed at compile time for the common configurations, the
// group and word arithmetic is shifts and constants. Other configurations,
// more rows, activations too large for LDS and unaligned inputs take a kernel
// that reads x from memory, one entry per lane at a time.
#include "device.hpp"
#include "kernels.hpp"

namespace e2m1 {
namespace {

constexpr int kThreads = 256;                 // generic kernel
constexpr int kWaves = kThreads / kWave;
constexpr int kFastWaves = 8;                 // fast kernel: waves per workgroup
constexpr int kFastThreads = kFastWaves * kWave;
constexpr int kChunks = 2;                    // 16-byte value chunks in flight per lane
constexpr size_t kMaxLdsBytes = 65536;        // staged activations per workgroup

__host__ __device__ constexpr int nm_bits(int m) { return m <= 2 ? 1 : m <= 4 ? 2 : m <= 8 ? 3 : 4; }

template <bool kBf16Out>
__device__ __forceinline__ void nm_store(void* y, int64_t idx, float v) {
    if constexpr (kBf16Out)
        reinterpret_cast<uint16_t*>(y)[idx] = (uint16_t)f32_to_bf16_rne(v);
    else
        reinterpret_cast<float*>(y)[idx] = v;
}

template <int NN, int MM, int BS>
struct NmGeo {
    static constexpr int kBits = nm_bits(MM);
    static constexpr int kPacking = 32 / kBits;
    static constexpr uint32_t kPosMask = (1u << kBits) - 1u;
    static constexpr int kSpan = 8 * MM / NN;              // columns covered by 8 consecutive entries
    static constexpr int kPad = BS == 4 ? 4 : 2;           // bf16 of padding after each staged span
    static constexpr int kSpanElems = kSpan * BS + kPad;   // staged bf16 per span
    static_assert(8 % NN == 0, "a chunk of 8 entries must hold whole groups");
};

template <int NN, int MM, int BS>
size_t nm_lds_bytes(int k) {
    using G = NmGeo<NN, MM, BS>;
    return (size_t)(k / G::kSpan) * G::kSpanElems * sizeof(uint16_t);
}

// Eight entries e0 .. e0 + 7 of one row: values v (bf16 pairs), positions in
// word m0 (and m1 for the entries past m0), x staged span by span in xs.
template <int NN, int MM, int B, int BS>
__device__ __forceinline__ void nm_chunk(const uint4 v, uint32_t m0, uint32_t m1, int e0, const uint16_t* xs,
                                         float (&acc)[B]) {
    using G = NmGeo<NN, MM, BS>;
    uint32_t p;   // the 8 positions, kBits each, entry i at bit kBits i
    if constexpr (G::kPacking % 8 == 0) {
        p = m0 >> (G::kBits * (e0 % G::kPacking));
    } else {
        constexpr int used = G::kPacking * G::kBits;
        const uint64_t s = (uint64_t)(m0 & ((1u << used) - 1u)) | ((uint64_t)m1 << used);
        p = (uint32_t)(s >> (G::kBits * (e0 % G::kPacking)));
    }
    const uint16_t* base = xs + (e0 >> 3) * G::kSpanElems;   // span e0 / 8 (its groups start at column e0 M / N)
    const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
        const uint32_t pa = (p >> (G::kBits * i)) & G::kPosMask;
        const uint32_t pb = (p >> (G::kBits * (i + 1))) & G::kPosMask;
        const uint16_t* xa = base + ((i / NN) * MM + (int)pa) * BS;
        const uint16_t* xb = base + (((i + 1) / NN) * MM + (int)pb) * BS;
        const uint32_t w = vv[i >> 1];
        if constexpr (BS == 1) {
            const u16x2 t = {xa[0], xb[0]};
            acc[0] = dot2_bf16(w, __builtin_bit_cast(uint32_t, t), acc[0]);
        } else if constexpr (BS == 2) {
            const uint32_t a = *reinterpret_cast<const uint32_t*>(xa), b = *reinterpret_cast<const uint32_t*>(xb);
            acc[0] = dot2_bf16(w, __builtin_amdgcn_perm(b, a, 0x05040100u), acc[0]);
            if constexpr (B > 1) acc[1] = dot2_bf16(w, __builtin_amdgcn_perm(b, a, 0x07060302u), acc[1]);
        } else {
            const uint2 a = *reinterpret_cast<const uint2*>(xa), b = *reinterpret_cast<const uint2*>(xb);
            acc[0] = dot2_bf16(w, __builtin_amdgcn_perm(b.x, a.x, 0x05040100u), acc[0]);
            if constexpr (B > 1) acc[1] = dot2_bf16(w, __builtin_amdgcn_perm(b.x, a.x, 0x07060302u), acc[1]);
            if constexpr (B > 2) acc[2] = dot2_bf16(w, __builtin_amdgcn_perm(b.y, a.y, 0x05040100u), acc[2]);
            if constexpr (B > 3) acc[3] = dot2_bf16(w, __builtin_amdgcn_perm(b.y, a.y, 0x07060302u), acc[3]);
        }
    }
}

// B activation rows in BS slots per column (BS = 1, 2 or 4, B <= BS). Requires
// per_row % 8 == 0 (so k is a whole number of spans), 16-byte aligned values
// and x, and the staged x within kMaxLdsBytes.
template <int NN, int MM, int B, int BS, bool kBf16Out>
__global__ __launch_bounds__(kFastThreads) void nm_spmm_kernel(const uint16_t* __restrict__ values,
                                                               const uint32_t* __restrict__ meta,
                                                               const uint16_t* __restrict__ x,
                                                               void* __restrict__ y, int rows, int k) {
    using G = NmGeo<NN, MM, BS>;
    extern __shared__ __attribute__((aligned(16))) uint16_t nm_x[];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int per_row = (k / MM) * NN;
    const int words = (per_row + G::kPacking - 1) / G::kPacking;

    // x -> LDS, 8 columns per item: column c of row b at (c / span) * kSpanElems + (c % span) * BS + b
    for (int i = threadIdx.x; i < k / 8; i += kFastThreads) {
        const int c = 8 * i;
        uint4 t[BS];
#pragma unroll
        for (int b = 0; b < BS; ++b)
            t[b] = b < B ? reinterpret_cast<const uint4*>(x + (size_t)b * k)[i] : make_uint4(0, 0, 0, 0);
        uint16_t* d = nm_x + (c / G::kSpan) * G::kSpanElems + (c % G::kSpan) * BS;
        if constexpr (BS == 1) {
            uint32_t* dw = reinterpret_cast<uint32_t*>(d);   // 4-byte aligned (spans are padded by 4 bytes)
            dw[0] = t[0].x;
            dw[1] = t[0].y;
            dw[2] = t[0].z;
            dw[3] = t[0].w;
        } else {
            const uint32_t r0[4] = {t[0].x, t[0].y, t[0].z, t[0].w};
            const uint32_t r1[4] = {t[1].x, t[1].y, t[1].z, t[1].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {   // columns c + 2 j and c + 2 j + 1
                const uint32_t lo01 = __builtin_amdgcn_perm(r1[j], r0[j], 0x05040100u);
                const uint32_t hi01 = __builtin_amdgcn_perm(r1[j], r0[j], 0x07060302u);
                // stores no wider than the padding keeps aligned: 4 bytes (BS = 2), 8 bytes (BS = 4)
                if constexpr (BS == 2) {
                    reinterpret_cast<uint32_t*>(d)[2 * j] = lo01;
                    reinterpret_cast<uint32_t*>(d)[2 * j + 1] = hi01;
                } else {
                    const uint32_t r2 = j == 0 ? t[2].x : j == 1 ? t[2].y : j == 2 ? t[2].z : t[2].w;
                    const uint32_t r3 = j == 0 ? t[3].x : j == 1 ? t[3].y : j == 2 ? t[3].z : t[3].w;
                    const uint32_t lo23 = __builtin_amdgcn_perm(r3, r2, 0x05040100u);
                    const uint32_t hi23 = __builtin_amdgcn_perm(r3, r2, 0x07060302u);
                    reinterpret_cast<uint2*>(d)[2 * j] = make_uint2(lo01, lo23);
                    reinterpret_cast<uint2*>(d)[2 * j + 1] = make_uint2(hi01, hi23);
                }
            }
        }
    }
    __syncthreads();

    const int full = per_row / (8 * kWave);   // chunks every lane of a row has
    for (int row = blockIdx.x * kFastWaves + wave; row < rows; row += gridDim.x * kFastWaves) {   // wave-uniform
        const uint16_t* vrow = values + (size_t)row * per_row + 8 * lane;
        const uint32_t* mrow = meta + (size_t)row * words;
        float acc[B];
#pragma unroll
        for (int b = 0; b < B; ++b) acc[b] = 0.f;
        int j = 0;
        for (; j + kChunks <= full; j += kChunks) {
            uint4 v[kChunks];
            uint32_t m0[kChunks], m1[kChunks];
#pragma unroll
            for (int u = 0; u < kChunks; ++u) {   // all loads first
                const int e0 = 8 * lane + 8 * kWave * (j + u);
                v[u] = load_nt16(vrow + 8 * kWave * (j + u));
                m0[u] = mrow[e0 / G::kPacking];
                m1[u] = G::kPacking % 8 != 0 ? mrow[min((e0 + 7) / G::kPacking, words - 1)] : 0u;
            }
#pragma unroll
            for (int u = 0; u < kChunks; ++u)
                nm_chunk<NN, MM, B, BS>(v[u], m0[u], m1[u], 8 * lane + 8 * kWave * (j + u), nm_x, acc);
        }
        for (; 8 * kWave * j + 8 * lane < per_row; ++j) {   // the rest, lanes past the row end idle
            const int e0 = 8 * lane + 8 * kWave * j;
            const uint4 v = load_nt16(vrow + 8 * kWave * j);
            const uint32_t m0 = mrow[e0 / G::kPacking];
            const uint32_t m1 = G::kPacking % 8 != 0 ? mrow[min((e0 + 7) / G::kPacking, words - 1)] : 0u;
            nm_chunk<NN, MM, B, BS>(v, m0, m1, e0, nm_x, acc);
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
    constexpr int BS = B == 1 ? 1 : B == 2 ? 2 : 4;
    const size_t lds = nm_lds_bytes<NN, MM, BS>(k);
    static int per_cu = 0;
    if (per_cu == 0) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(nm_spmm_kernel<NN, MM, B, BS, kBf16Out>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLdsBytes);
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, nm_spmm_kernel<NN, MM, B, BS, kBf16Out>,
                                                         kFastThreads, kMaxLdsBytes / 2) != hipSuccess ||
            per_cu < 1)
            per_cu = 1;
    }
    // occupancy taken at half the LDS limit; larger stagings simply fit fewer workgroups per CU
    const int want = (rows + kFastWaves - 1) / kFastWaves;
    const int grid = min(want, per_cu * device_cu_count());
    nm_spmm_kernel<NN, MM, B, BS, kBf16Out><<<grid, kFastThreads, lds, stream>>>(values, meta, x, y, rows, k);
    return hipGetLastError();
}

template <int NN, int MM, int B>
bool nm_fits(int k) {
    constexpr int BS = B == 1 ? 1 : B == 2 ? 2 : 4;
    return k % NmGeo<NN, MM, BS>::kSpan == 0 && nm_lds_bytes<NN, MM, BS>(k) <= kMaxLdsBytes;
}

template <int NN, int MM, bool kBf16Out>
bool try_fast(int batch, const uint16_t* values, const uint32_t* meta, const uint16_t* x, void* y, int rows, int k,
              hipStream_t stream, hipError_t* err) {
    switch (batch) {
        case 1:
            if (!nm_fits<NN, MM, 1>(k)) return false;
            *err = run_nm<NN, MM, 1, kBf16Out>(values, meta, x, y, rows, k, stream);
            return true;
        case 2:
            if (!nm_fits<NN, MM, 2>(k)) return false;
            *err = run_nm<NN, MM, 2, kBf16Out>(values, meta, x, y, rows, k, stream);
            return true;
        case 3:
            if (!nm_fits<NN, MM, 3>(k)) return false;
            *err = run_nm<NN, MM, 3, kBf16Out>(values, meta, x, y, rows, k, stream);
            return true;
        case 4:
            if (!nm_fits<NN, MM, 4>(k)) return false;
            *err = run_nm<NN, MM, 4, kBf16Out>(values, meta, x, y, rows, k, stream);
            return true;
        default: return false;
    }
}

template <bool kBf16Out>
hipError_t launch_nm_t(const uint16_t* values, const uint32_t* meta, const uint16_t* x, void* y, int batch,
                       int rows, int k, int nn, int mm, hipStream_t stream) {
    const int per_row = (k / mm) * nn;
    const bool aligned = per_row % 8 == 0 && (reinterpret_cast<uintptr_t>(values) & 15u) == 0 &&
                         (reinterpret_cast<uintptr_t>(x) & 15u) == 0;
    hipError_t err = hipSuccess;
    if (aligned) {
        if (nn == 2 && mm == 4 && try_fast<2, 4, kBf16Out>(batch, values, meta, x, y, rows, k, stream, &err)) return err;
        if (nn == 1 && mm == 4 && try_fast<1, 4, kBf16Out>(batch, values, meta, x, y, rows, k, stream, &err)) return err;
        if (nn == 4 && mm == 8 && try_fast<4, 8, kBf16Out>(batch, values, meta, x, y, rows, k, stream, &err)) return err;
        if (nn == 1 && mm == 2 && try_fast<1, 2, kBf16Out>(batch, values, meta, x, y, rows, k, stream, &err)) return err;
        if (nn == 8 && mm == 16 && try_fast<8, 16, kBf16Out>(batch, values, meta, x, y, rows, k, stream, &err))
            return err;
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
