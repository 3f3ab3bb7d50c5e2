// platform_probe.hip -- the platform limits a per-launch roofline figure is
// read against, measured with the simplest possible kernels: the time of an
// empty launch, the time to stream B bytes from HBM with nothing else to do,
// a kernel that keeps every SIMD's matrix core busy (the reference point for
// the MFMA-busy counter; two instruction shapes), and the LDS read rate of a
// lane -> address pattern. Built into libe2m1probe.so (separate from
// libe2m1lut.so, which never loads it) and run by the benchmark's probe
// workloads.
//
// C entry points (the benchmark calls them through ctypes):
//
//   int e2m1_probe_empty(int64_t grid, int block, void* stream)
//       Launches an empty kernel of `grid` workgroups of `block` threads
//       (block 64 or 256, 1 <= grid < 2^31).
//
//   int64_t e2m1_probe_stream_grid(int64_t bytes, int block)
//       The grid e2m1_probe_stream launches for `bytes` (-1 if invalid).
//
//   int e2m1_probe_stream(const void* src, int64_t bytes, uint32_t* out,
//                         int64_t out_words, int block, int store, void* stream)
//       Reads `bytes` (a positive multiple of 16) from the device buffer
//       `src` with 16-byte non-temporal loads: each thread issues all eight
//       of its loads first, and load j of a wave covers 1 KB of consecutive
//       bytes. With store = 0 nothing is written (a store guarded by a
//       checksum test no input meets keeps the loads live); with store = 1
//       every wave writes one 4-byte checksum to out[wave] (out_words must
//       be at least grid * block / 64): a small output like a GEMV's; with
//       store = 2 only the first wave of the grid writes (out[0]).
//
//   int e2m1_probe_mfma(int64_t grid, int iters, int form, float* out,
//                       int64_t out_words, void* stream)
//       grid workgroups of four waves; every wave runs `iters` rounds of four
//       independent MFMA chains on register operands, then writes one float
//       per thread to out (out_words >= grid * 256). form 32:
//       v_mfma_f32_32x32x16_bf16 (32768 flops each), form 16:
//       v_mfma_f32_16x16x32_bf16 (16384 flops each). Flops per launch:
//       grid * 4 * iters * 4 * (flops of one instruction).
//
//   int e2m1_probe_expand(const void* src, int64_t src_bytes, void* dst,
//                         void* stream)
//       Reads src_bytes (a positive multiple of 16) with 16-byte non-temporal
//       loads and writes four times as many bytes to dst: 16-byte chunk j of
//       src (bitwise inverted) goes to chunk j of each of the four
//       src_bytes-long planes of dst, with non-temporal stores, so every load
//       and store instruction of a wave covers 1 KB of consecutive bytes;
//       each thread issues its eight loads first. The byte ratio of a 4-bit
//       code to its bf16 decode (1 : 4): the streaming reference of the
//       write-heavy kernels.
//
//   int e2m1_probe_lds(const uint32_t* table, int64_t grid, int iters,
//                      uint32_t* out, int64_t out_words, void* stream)
//       grid workgroups of eight waves; lane l of every wave reads the
//       16-byte LDS slot table[l] % 4096 (of a 64 KiB array) 8 * iters times
//       with ds_read_b128, eight reads back to back per wait, then writes one
//       word per thread to out (out_words >= grid * 512). LDS bytes read per
//       launch: grid * 512 * 16 * 8 * iters. `table` holds 64 words.
//
// All return 0, or -1 for an argument out of range, -2 for a launch error.
// Every index is clamped to the buffer, so every access is in bounds.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kLoads = 8;
constexpr uint32_t kNever = 0x9E3779B9u;

template <int kBlock>
__global__ __launch_bounds__(kBlock) void probe_empty_kernel() {}

template <int kBlock, int kStore>
__global__ __launch_bounds__(kBlock) void probe_stream_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                              uint32_t* __restrict__ out) {
    const int64_t base = (int64_t)blockIdx.x * kLoads * kBlock + threadIdx.x;
    u32x4 v[kLoads];
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
        const int64_t i = base + (int64_t)j * kBlock;
        v[j] = __builtin_nontemporal_load(src + (i < n16 ? i : n16 - 1));
    }
    __builtin_amdgcn_sched_barrier(0);  // every load is issued before the first wait
    uint32_t acc = 0;
#pragma unroll
    for (int j = 0; j < kLoads; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    if constexpr (kStore == 1) {
        for (int d = 32; d >= 1; d >>= 1) acc ^= __shfl_xor(acc, d, 64);
        if ((threadIdx.x & 63) == 0) out[(int64_t)blockIdx.x * (kBlock / 64) + threadIdx.x / 64] = acc;
    } else if constexpr (kStore == 2) {
        for (int d = 32; d >= 1; d >>= 1) acc ^= __shfl_xor(acc, d, 64);
        if (blockIdx.x == 0 && threadIdx.x == 0) out[0] = acc;
        else if (acc == kNever) out[0] = acc;
    } else {
        if (acc == kNever) out[0] = acc;
    }
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int kForm>
__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters, float* __restrict__ out) {
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)((float)((threadIdx.x + i) & 7) * 0.125f);
        b[i] = (__bf16)((float)((threadIdx.x * 3 + i) & 7) * -0.0625f);
    }
    float total = 0.f;
    if constexpr (kForm == 32) {
        f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
        for (int it = 0; it < iters; ++it) {
            c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
        }
        const f32x16 t = c0 + c1 + c2 + c3;
#pragma unroll
        for (int e = 0; e < 16; ++e) total += t[e];
    } else {
        // written out: with the builtin the compiler shuffles these four accumulators through
        // extra registers every round, which the probe would time instead of the instruction
        f32x4 c0 = {}, c1 = {}, c2 = {}, c3 = {};
        for (int it = 0; it < iters; ++it) {
            asm volatile(
                "v_mfma_f32_16x16x32_bf16 %0, %4, %5, %0\n"
                "v_mfma_f32_16x16x32_bf16 %1, %4, %5, %1\n"
                "v_mfma_f32_16x16x32_bf16 %2, %4, %5, %2\n"
                "v_mfma_f32_16x16x32_bf16 %3, %4, %5, %3\n"
                : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3)
                : "v"(a), "v"(b));
        }
        const f32x4 t = c0 + c1 + c2 + c3;
#pragma unroll
        for (int e = 0; e < 4; ++e) total += t[e];
    }
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = total;
}

// Read one 16-byte chunk, write it to four planes: eight chunks per thread, every load first.
__global__ __launch_bounds__(256) void probe_expand_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                           u32x4* __restrict__ dst) {
    const int64_t base = (int64_t)blockIdx.x * kLoads * 256 + threadIdx.x;
    u32x4 v[kLoads];
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
        const int64_t i = base + (int64_t)j * 256;
        v[j] = __builtin_nontemporal_load(src + (i < n16 ? i : n16 - 1));
    }
    __builtin_amdgcn_sched_barrier(0);
    // chunks past the end (the grid's tail) rewrite the last chunk with its own value: no branch
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
        const int64_t i = base + (int64_t)j * 256;
        const u32x4 w = ~v[j];
        u32x4* d = dst + (i < n16 ? i : n16 - 1);
#pragma unroll
        for (int q = 0; q < 4; ++q) __builtin_nontemporal_store(w, d + q * n16);
    }
}

// Eight ds_read_b128 of one address per round, one wait per round: the reads
// of a round are in flight together, so the time per round is set by the LDS
// read rate of the pattern (with eight waves per workgroup sharing the LDS).
__global__ __launch_bounds__(512) void probe_lds_kernel(const uint32_t* __restrict__ table, int iters,
                                                        uint32_t* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) uint32_t lds[16384];   // the kernel's only LDS variable: address 0
    for (int i = threadIdx.x; i < 16384; i += 512) lds[i] = (uint32_t)i * 2654435761u;
    __syncthreads();
    const int l = threadIdx.x & 63;
    const uint32_t a = (table[l] % 4096u) * 16u;   // byte address of the lane's slot
    uint32_t acc = 0;
    for (int it = 0; it < iters; ++it) {
        uint32_t x0, x1, x2, x3;
        asm volatile(
            "ds_read_b128 v[100:103], %4\n"
            "ds_read_b128 v[104:107], %4\n"
            "ds_read_b128 v[108:111], %4\n"
            "ds_read_b128 v[112:115], %4\n"
            "ds_read_b128 v[116:119], %4\n"
            "ds_read_b128 v[120:123], %4\n"
            "ds_read_b128 v[124:127], %4\n"
            "ds_read_b128 v[128:131], %4\n"
            "s_waitcnt lgkmcnt(0)\n"
            "v_mov_b32 %0, v100\n"
            "v_mov_b32 %1, v105\n"
            "v_mov_b32 %2, v110\n"
            "v_mov_b32 %3, v131\n"
            : "=v"(x0), "=v"(x1), "=v"(x2), "=v"(x3)
            : "v"(a)
            : "memory", "v100", "v101", "v102", "v103", "v104", "v105", "v106", "v107", "v108", "v109", "v110",
              "v111", "v112", "v113", "v114", "v115", "v116", "v117", "v118", "v119", "v120", "v121", "v122",
              "v123", "v124", "v125", "v126", "v127", "v128", "v129", "v130", "v131");
        acc ^= x0 ^ x1 ^ x2 ^ x3;
    }
    // keeps the array (and so its LDS allocation) live: the reads above are opaque to the compiler
    out[(int64_t)blockIdx.x * 512 + threadIdx.x] = acc + lds[(threadIdx.x * 7) & 16383];
}

int64_t stream_grid(int64_t bytes, int block) {
    if (bytes <= 0 || bytes % 16 != 0 || (block != 64 && block != 256)) return -1;
    const int64_t per = (int64_t)kLoads * block;
    const int64_t grid = (bytes / 16 + per - 1) / per;
    return grid < ((int64_t)1 << 31) ? grid : -1;
}

}  // namespace

extern "C" int e2m1_probe_empty(int64_t grid, int block, void* stream) {
    if (grid < 1 || grid >= ((int64_t)1 << 31)) return -1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (block == 64) probe_empty_kernel<64><<<dim3((unsigned)grid), dim3(64), 0, s>>>();
    else if (block == 256) probe_empty_kernel<256><<<dim3((unsigned)grid), dim3(256), 0, s>>>();
    else return -1;
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

extern "C" int64_t e2m1_probe_stream_grid(int64_t bytes, int block) { return stream_grid(bytes, block); }

extern "C" int e2m1_probe_stream(const void* src, int64_t bytes, uint32_t* out, int64_t out_words, int block,
                                 int store, void* stream) {
    const int64_t grid = stream_grid(bytes, block);
    if (grid < 0 || src == nullptr || out == nullptr || out_words < 1) return -1;
    if (store < 0 || store > 2 || (store == 1 && out_words < grid * (block / 64))) return -1;
    const u32x4* p = static_cast<const u32x4*>(src);
    const int64_t n16 = bytes / 16;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 g((unsigned)grid);
    if (block == 64) {
        if (store == 1) probe_stream_kernel<64, 1><<<g, dim3(64), 0, s>>>(p, n16, out);
        else if (store == 2) probe_stream_kernel<64, 2><<<g, dim3(64), 0, s>>>(p, n16, out);
        else probe_stream_kernel<64, 0><<<g, dim3(64), 0, s>>>(p, n16, out);
    } else {
        if (store == 1) probe_stream_kernel<256, 1><<<g, dim3(256), 0, s>>>(p, n16, out);
        else if (store == 2) probe_stream_kernel<256, 2><<<g, dim3(256), 0, s>>>(p, n16, out);
        else probe_stream_kernel<256, 0><<<g, dim3(256), 0, s>>>(p, n16, out);
    }
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

extern "C" int e2m1_probe_mfma(int64_t grid, int iters, int form, float* out, int64_t out_words, void* stream) {
    if (grid < 1 || grid >= ((int64_t)1 << 31) || iters < 1 || out == nullptr || out_words < grid * 256) return -1;
    if (form != 16 && form != 32) return -1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (form == 32) probe_mfma_kernel<32><<<dim3((unsigned)grid), dim3(256), 0, s>>>(iters, out);
    else probe_mfma_kernel<16><<<dim3((unsigned)grid), dim3(256), 0, s>>>(iters, out);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

extern "C" int e2m1_probe_expand(const void* src, int64_t src_bytes, void* dst, void* stream) {
    if (src == nullptr || dst == nullptr || src_bytes <= 0 || src_bytes % 16 != 0) return -1;
    const int64_t n16 = src_bytes / 16;
    const int64_t grid = (n16 + (int64_t)kLoads * 256 - 1) / ((int64_t)kLoads * 256);
    if (grid >= ((int64_t)1 << 31)) return -1;
    probe_expand_kernel<<<dim3((unsigned)grid), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const u32x4*>(src), n16, static_cast<u32x4*>(dst));
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

extern "C" int e2m1_probe_lds(const uint32_t* table, int64_t grid, int iters, uint32_t* out, int64_t out_words,
                              void* stream) {
    if (table == nullptr || out == nullptr || grid < 1 || grid >= ((int64_t)1 << 31) || iters < 1 ||
        out_words < grid * 512)
        return -1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    probe_lds_kernel<<<dim3((unsigned)grid), dim3(512), 0, s>>>(table, iters, out);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}
