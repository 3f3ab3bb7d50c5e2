// gemm.hip -- MXFP4 weight GEMM for many activation rows (dequant_gemm): the
// prefill counterpart of dequant_gemv.
//
// Semantics: y[m][n] = sum_k dec(W)[n][k] x[m][k] with fp32 accumulation, W
// MXFP4 (E2M1 codes + one E8M0 scale per 32 columns, the unpack of the vLLM
// pull request 51583 digest, section "功能与动机"), x bf16. The digest's
// comment section describes the CPU GEMM decoding each weight block into a
// bf16 tile before the multiply ("decode to tile"); here the decode feeds the
// matrix cores directly.
//
// gfx950 design. With hundreds of activation rows the product is bound by
// the matrix cores (2 m flops per 0.53 bytes of weights), so the kernel is a
// tiled bf16 MFMA GEMM whose weight operand is decoded on the way in. Two
// forms share the MFMA work: the direct-to-LDS form (K % 64 == 0, below the
// first) copies each step's tiles into LDS with buffer_load ... lds, and the
// register form here serves any K % 32 == 0:
//   * A workgroup of four waves owns a tile of 128 weight rows x 128
//     activation rows and walks K in steps of 64 columns. Each step, its
//     threads copy the step's x tile (128 x 64 bf16) and the raw code lines
//     (128 rows x 32 bytes) and scale bytes of W into LDS with 16-byte loads.
//     The code lines are read with ordinary (cached) loads: each weight tile
//     is read again by every activation-row tile, and a non-temporal hint
//     cost 30 % here. Two register sets carry the copies: the loads of step s + 2 are issued
//     before the MFMAs of step s, the registers of step s + 1 (requested a
//     step earlier) are written to the other LDS buffer after them, one
//     barrier per step. x and the scales are read through buffer resources:
//     plain loads through their restrict pointers were sunk by the compiler
//     next to their first use, exposing the full load latency every step.
//   * Waves are laid out 2 x 2 over the tile; each owns 64 weight rows x 64
//     activation rows as 2 x 2 tiles of v_mfma_f32_32x32x16_bf16 (each
//     operand register then serves twice the flops of a 16 x 16 x 32 one, and
//     back-to-back independent 32 x 32 x 16 MFMAs run about 10 % faster on
//     this part). Lane l = 32 g + r takes 8 codes (4 bytes) of weight row r
//     per 16-column slice and decodes them with four
//     v_cvt_scalef32_pk_bf16_fp4 (two codes each, table lookup and E8M0 scale
//     in one instruction); each decoded A operand serves two MFMAs. B
//     operands are 16-byte LDS reads of x at the same columns.
//   * D element (weight row 8 p + 4 g + j, activation row c) sits in
//     component 4 p + j of lane 32 g + c, so each lane stores runs of four
//     consecutive outputs of one row of y.
// Rows past N or M are loaded clamped and not stored; a 32-column block past
// K is decoded as zero weights.
#include "device.hpp"
#include "kernels.hpp"

namespace e2m1 {
namespace {

constexpr int kThreads = 256;
constexpr int kTileN = 128;                  // weight rows per workgroup
constexpr int kTileM = 128;                  // activation rows per workgroup
constexpr int kStepK = 64;                   // columns per step
constexpr int kXPitch = kStepK + 8;          // bf16 per staged x row (16-byte pad spreads the banks)
constexpr int kWPitch = 32 + 4;              // bytes per staged code row
constexpr int kXElems = kTileM * kXPitch;
constexpr int kWBytes = kTileN * kWPitch;
constexpr int kXChunks = kTileM * kStepK / 8 / kThreads;   // 16-byte x chunks per thread per step

typedef float f32x16 __attribute__((ext_vector_type(16)));

struct GemmBuf {
    uint16_t x[kXElems];
    uint8_t w[kWBytes];
    uint8_t s[kThreads * 2];   // rows < kTileN are read; every thread stores (an unconditional store keeps
                               // the scale loads where they are issued)
};

template <bool kBf16Out>
__device__ __forceinline__ void store4(void* y, int64_t idx, const f32x4& v, bool full, int count) {
    if constexpr (kBf16Out) {
        uint16_t* p = reinterpret_cast<uint16_t*>(y) + idx;
        if (full && (idx & 3) == 0) {
            *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        } else {
            for (int j = 0; j < count; ++j) p[j] = (uint16_t)f32_to_bf16_rne(v[j]);
        }
    } else {
        float* p = reinterpret_cast<float*>(y) + idx;
        if (full && (idx & 3) == 0) {
            *reinterpret_cast<f32x4*>(p) = v;
        } else {
            for (int j = 0; j < count; ++j) p[j] = v[j];
        }
    }
}

// Three waves per SIMD (three workgroups per compute unit: 47 KB of LDS each)
// caps the kernel at 168 VGPRs; left alone, the compiler takes 224 and fits two.
template <bool kBf16Out>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void gemm_kernel(const uint8_t* __restrict__ packed,
                                                        const uint8_t* __restrict__ scales,
                                                        const uint16_t* __restrict__ x, void* __restrict__ y,
                                                        int m_rows, int n, int kc) {
    __shared__ __attribute__((aligned(16))) GemmBuf buf[2];
    const int t = threadIdx.x;
    const int lane = t & (kWave - 1);
    const int wave = t / kWave;
    const int r32 = lane & 31, g2 = lane >> 5;
    const int wn = (wave & 1) * 64, wm = (wave >> 1) * 64;   // the wave's quarter of the tile
    const int K = kc * 32;
    const int nsteps = (kc + 1) / 2;
    const int ntn = (n + kTileN - 1) / kTileN;
    const int n0 = (blockIdx.x % ntn) * kTileN;
    const int m0 = (blockIdx.x / ntn) * kTileM;

    // this thread's share of a step's copies: x chunks t + 256 i (row id / 8, 8 columns each),
    // code line t (row t / 2, 32-column block t % 2), scale bytes of row t % 128
    // resources over this tile's rows only, so every offset is below 128 k * 2 bytes
    const int mt = min(kTileM, m_rows - m0), nt = min(kTileN, n - n0);
    const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(x + (size_t)m0 * K), 0, mt * K * 2, kBufferWord3);
    const __amdgpu_buffer_rsrc_t sres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(scales + (size_t)n0 * kc), 0, nt * kc, kBufferWord3);
    uint32_t xoff[kXChunks];
#pragma unroll
    for (int i = 0; i < kXChunks; ++i) xoff[i] = 2u * (uint32_t)min((t + kThreads * i) >> 3, mt - 1) * (uint32_t)K;
    const uint32_t soff = (uint32_t)min(t % kTileN, nt - 1) * (uint32_t)kc;
    const int xcol = 8 * (t & 7);   // the same for every chunk (kThreads is a multiple of 8)
    const uint8_t* wsrc = packed + (size_t)min(n0 + (t >> 1), n - 1) * (K / 2);

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    uint4 xr[2][kXChunks], wr[2];
    uint32_t s0[2], s1[2];   // a step's two scale bytes, combined only when staged
// Step `st`'s copies into register set p. Columns past K (the second block of
// a last half step) read the row's last 8 columns: finite values that meet
// zero weights.
#define E2M1_GEMM_ISSUE(st, p)                                                                          \
    {                                                                                                   \
        const int c0 = (st) * kStepK;                                                                   \
        _Pragma("unroll") for (int i = 0; i < kXChunks; ++i) {                                          \
            const u32x4 v_ = __builtin_amdgcn_raw_buffer_load_b128(                                     \
                xres, xoff[i] + 2u * (uint32_t)min(c0 + xcol, K - 8), 0, 0);                            \
            xr[p][i] = make_uint4(v_[0], v_[1], v_[2], v_[3]);                                          \
        }                                                                                               \
        wr[p] = *reinterpret_cast<const uint4*>(wsrc + (size_t)min(2 * (st) + (t & 1), kc - 1) * 16);    \
        s0[p] = __builtin_amdgcn_raw_buffer_load_b8(sres, soff + (uint32_t)min(2 * (st), kc - 1), 0, 0);     \
        s1[p] = __builtin_amdgcn_raw_buffer_load_b8(sres, soff + (uint32_t)min(2 * (st) + 1, kc - 1), 0, 0); \
    }
// Register set p (step `st`) into LDS buffer bb; a block past K is staged as zero codes.
#define E2M1_GEMM_STAGE(bb, st, p)                                                                      \
    {                                                                                                   \
        _Pragma("unroll") for (int i = 0; i < kXChunks; ++i) {                                          \
            const int id = t + kThreads * i;                                                            \
            *reinterpret_cast<uint4*>((bb).x + (id >> 3) * kXPitch + 8 * (id & 7)) = xr[p][i];          \
        }                                                                                               \
        const uint32_t keep = 2 * (st) + (t & 1) < kc ? 0xFFFFFFFFu : 0u;                               \
        uint32_t* wd = reinterpret_cast<uint32_t*>((bb).w + (t >> 1) * kWPitch + 16 * (t & 1));          \
        wd[0] = wr[p].x & keep;                                                                         \
        wd[1] = wr[p].y & keep;                                                                         \
        wd[2] = wr[p].z & keep;                                                                         \
        wd[3] = wr[p].w & keep;                                                                         \
        *reinterpret_cast<uint16_t*>((bb).s + 2 * t) = (uint16_t)(s0[p] | (s1[p] << 8));                \
    }
// The MFMAs of the step held in buffer bb: 16-column slices q, lane group g2
// taking columns 16 q + 8 g2 .. + 7 of both operands.
#define E2M1_GEMM_COMPUTE(bb)                                                                           \
    {                                                                                                   \
        _Pragma("unroll") for (int q = 0; q < 4; ++q) {                                                 \
            bf16x8 a[2];                                                                                \
            _Pragma("unroll") for (int i = 0; i < 2; ++i) {                                             \
                const int row = wn + 32 * i + r32;                                                      \
                const uint32_t codes = *reinterpret_cast<const uint32_t*>((bb).w + row * kWPitch + 8 * q + 4 * g2); \
                const float sc = e8m0_scale((bb).s[2 * row + (q >> 1)]);                                \
                const u32x4 u = {fp4x2_to_bf16x2<0>(codes, sc), fp4x2_to_bf16x2<1>(codes, sc),          \
                                 fp4x2_to_bf16x2<2>(codes, sc), fp4x2_to_bf16x2<3>(codes, sc)};         \
                a[i] = __builtin_bit_cast(bf16x8, u);                                                   \
            }                                                                                           \
            _Pragma("unroll") for (int j = 0; j < 2; ++j) {                                             \
                const bf16x8 bx = *reinterpret_cast<const bf16x8*>((bb).x + (wm + 32 * j + r32) * kXPitch + \
                                                                   16 * q + 8 * g2);                    \
                _Pragma("unroll") for (int i = 0; i < 2; ++i)                                           \
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bx, acc[i][j], 0, 0, 0);  \
            }                                                                                           \
        }                                                                                               \
    }
// Step `step` with parity p: request step + 2 into register set p (free since
// its step was staged), compute from buffer p, stage register set 1 - p (step
// + 1) into buffer 1 - p (every wave finished reading it before the last barrier).
// The last steps re-request their own copies, staged into the idle buffer and never read.
#define E2M1_GEMM_STEP(step, p)                                                                         \
    {                                                                                                   \
        E2M1_GEMM_ISSUE(min((step) + 2, nsteps - 1), p)                                                 \
        asm volatile("" ::: "memory");   /* the loads stay here, ahead of the step's MFMAs */           \
        __builtin_amdgcn_sched_barrier(0);                                                              \
        E2M1_GEMM_COMPUTE(buf[p])                                                                       \
        __builtin_amdgcn_sched_barrier(0);   /* the staging (and its waits) stays after them */         \
        E2M1_GEMM_STAGE(buf[1 - (p)], min((step) + 1, nsteps - 1), 1 - (p))                             \
        __syncthreads();                                                                                \
    }

    E2M1_GEMM_ISSUE(0, 0)
    E2M1_GEMM_STAGE(buf[0], 0, 0)
    E2M1_GEMM_ISSUE(min(1, nsteps - 1), 1)
    __syncthreads();
    for (int s = 0; s < nsteps; s += 2) {   // unrolled by two: register sets and buffers are static
        E2M1_GEMM_STEP(s, 0)
        if (s + 1 < nsteps) E2M1_GEMM_STEP(s + 1, 1)   // workgroup-uniform
    }
#undef E2M1_GEMM_STEP
#undef E2M1_GEMM_COMPUTE
#undef E2M1_GEMM_STAGE
#undef E2M1_GEMM_ISSUE

    // lane l = 32 g2 + c holds, for tile (i, j) and p < 4, rows n0 + wn + 32 i + 8 p + 4 g2 .. + 3
    // of activation row m0 + wm + 32 j + c (accumulator components 4 p .. 4 p + 3)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int m = m0 + wm + 32 * j + r32;
        if (m >= m_rows) continue;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int nn = n0 + wn + 32 * i + 8 * p + 4 * g2;
                if (nn >= n) continue;
                const int count = min(4, n - nn);
                const f32x4 v = {acc[i][j][4 * p], acc[i][j][4 * p + 1], acc[i][j][4 * p + 2], acc[i][j][4 * p + 3]};
                store4<kBf16Out>(y, (int64_t)m * n + nn, v, count == 4, count);
            }
    }
}

// ---------------------------------------------------- direct-to-LDS form --
//
// Eight waves on a tile of 256 weight rows x 128 activation rows (4 x 2
// waves, each 64 x 64 as 2 x 2 v_mfma_f32_32x32x16_bf16, as above), with
// every per-step copy made by the memory pipeline itself: buffer_load ... lds
// writes each lane's 2, 4 or 16 bytes straight into LDS (lane l of an
// instruction at base + max(size, 4) * l), so no register holds a copy and no
// ds_write stages one, and the x tile of a step serves twice the weight rows.
// kStages LDS buffers rotate; step s + kStages - 1 is requested right after
// the barrier that opens step s (its buffer was last read in step s - 1).
// Steps are kSK = 64 columns (80 KB of LDS, two workgroups per compute unit)
// or 128 (150 KB, fewer barriers per flop) columns. The layouts are chosen
// through the lanes' source addresses:
//   * x: 16-byte chunk c of row r at slot c ^ (r / 2 % 8) (64 columns) or
//     c ^ (r % 16) (128) of its row, so a B-operand read (16 rows x one
//     chunk per 16 lanes) touches 16 different bank groups;
//   * codes: word j of a row's kSK / 2 bytes at slot j ^ (r / R % W), R rows
//     per 256-byte request and W words per row;
//   * scales: 2-byte loads (two 32-column blocks), which the memory pipeline
//     writes zero-extended into a 4-byte slot per lane.
// The compiler does not see these loads (inline asm, which also keeps them in
// place): every wave waits for its own with s_waitcnt vmcnt before the
// barrier, and requests past the last step read out of range (zeros, no
// memory access), so the count is the same every step, and the last wait
// drains them before the workgroup's LDS is released.

// lane's kBytes (2, 4 or 16) at byte offset voff of the buffer -> LDS lds + max(kBytes, 4) * lane
// (two bytes land zero-extended in a 4-byte slot). The LDS address goes through M0, which the asm
// sets itself; nothing else in these kernels uses M0.
template <int kBytes>
__device__ __forceinline__ void lds_load(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t lds) {
    if constexpr (kBytes == 16)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                     :: "s"(lds), "v"(voff), "s"(rsrc) : "memory");
    else if constexpr (kBytes == 4)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                     :: "s"(lds), "v"(voff), "s"(rsrc) : "memory");
    else
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_ushort %1, %2, 0 offen lds"
                     :: "s"(lds), "v"(voff), "s"(rsrc) : "memory");
}

template <int kN>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(kN) : "memory");
}

constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;   // a buffer offset past any resource's range

// kWN waves along the weight rows (tile of 64 kWN rows) x 2 along the activation rows (128);
// steps of kSK columns (64 or 128).
template <int kWN, int kSK>
struct GemmDmaBuf {
    static constexpr int kRows = 64 * kWN;
    uint16_t x[kTileM * kSK];               // [row][kSK], 16-byte chunks swizzled
    uint32_t w[kRows * (kSK / 8)];          // [row][kSK / 8 words], words swizzled
    uint32_t s[2 * kWN][kWave];             // [wave][lane]: scale pairs of rows 32 wave + lane % 32
};

template <bool kBf16Out, int kStages, int kWN, int kSK>
__global__ __launch_bounds__(128 * kWN) void gemm_dma_kernel(const uint8_t* __restrict__ packed,
                                                             const uint8_t* __restrict__ scales,
                                                             const uint16_t* __restrict__ x, void* __restrict__ y,
                                                             int m_rows, int n, int kc) {
    constexpr int kRows = 64 * kWN;                 // weight rows per tile
    constexpr int kChunks = kSK / 8;                // 16-byte x chunks per row and step (8 or 16)
    constexpr int kWords = kSK / 8;                 // 4-byte code words per row and step (8 or 16)
    constexpr int kXRowsPer = 1024 / (2 * kSK);     // x rows per 1 KB request
    constexpr int kXLoads = kTileM / kXRowsPer / (2 * kWN);          // per wave and step
    constexpr int kWRowsPer = 64 / kWords;          // code rows per 256-byte request
    constexpr int kWLoads = kRows / kWRowsPer / (2 * kWN);           // per wave and step
    constexpr int kPerStep = kXLoads + kWLoads + 1;                  // + one scale request
    constexpr int kQ = kSK / 16;                    // 16-column slices per step
    static_assert(kXLoads * kXRowsPer * 2 * kWN == kTileM && kWLoads * kWRowsPer * 2 * kWN == kRows, "requests");
    __shared__ __attribute__((aligned(16))) GemmDmaBuf<kWN, kSK> buf[kStages];
    const int t = threadIdx.x;
    const int lane = t & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(t / kWave);
    const int r32 = lane & 31, g2 = lane >> 5;
    const int wn = (wave % kWN) * 64, wm = (wave / kWN) * 64;
    const int K = kc * 32;
    const int nsteps = K / kSK;
    const int ntn = (n + kRows - 1) / kRows;
    const int n0 = (blockIdx.x % ntn) * kRows;
    const int m0 = (blockIdx.x / ntn) * kTileM;
    const int mt = min(kTileM, m_rows - m0), nt = min(kRows, n - n0);
    const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(x + (size_t)m0 * K), 0, mt * K * 2, kBufferWord3);
    const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(packed + (size_t)n0 * (K / 2)), 0, nt * (K / 2), kBufferWord3);
    const __amdgpu_buffer_rsrc_t sres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(scales + (size_t)n0 * kc), 0, nt * kc, kBufferWord3);

    // x: chunk c of row r at slot c ^ (r % kChunks) (kSK = 128) or c ^ (r / 2 % 8) (kSK = 64);
    // codes: word j of row r at slot j ^ (r / kWRowsPer % kWords); both spread the 16 rows of a
    // 16-lane read over the banks
    auto xswz = [](int r) __attribute__((always_inline)) { return kChunks == 16 ? (r & 15) : ((r >> 1) & 7); };
    auto wswz = [](int r) __attribute__((always_inline)) { return (r / kWRowsPer) % kWords; };
    uint32_t xoff[kXLoads], woff[kWLoads];
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) {
        const int row = kXRowsPer * (kXLoads * wave + i) + lane / kChunks, slot = lane % kChunks;
        xoff[i] = 2u * ((uint32_t)min(row, mt - 1) * (uint32_t)K + 8u * (uint32_t)(slot ^ xswz(row)));
    }
#pragma unroll
    for (int i = 0; i < kWLoads; ++i) {
        const int row = kWRowsPer * (kWLoads * wave + i) + lane / kWords, slot = lane % kWords;
        woff[i] = (uint32_t)min(row, nt - 1) * (uint32_t)(K / 2) + 4u * (uint32_t)(slot ^ wswz(row));
    }
    // scales: lane l takes row 32 wave + l % 32, bytes 2 (l / 32) .. + 1 of its kSK / 32 per step
    // (kSK = 64: only lanes < 32 load)
    const uint32_t soff = (uint32_t)min(32 * wave + r32, nt - 1) * (uint32_t)kc + 2u * (uint32_t)g2;
    const bool slane = kSK == 128 || lane < 32;
    auto issue = [&](int st, int stage) __attribute__((always_inline)) {
        const bool live = st < nsteps;
        GemmDmaBuf<kWN, kSK>& b = buf[stage];
        const uint32_t xb = (uint32_t)(uintptr_t)&b.x[0], wb = (uint32_t)(uintptr_t)&b.w[0];
#pragma unroll
        for (int i = 0; i < kXLoads; ++i)
            lds_load<16>(xres, live ? xoff[i] + 2u * kSK * (uint32_t)st : kOutOfRange,
                         __builtin_amdgcn_readfirstlane(xb + 1024u * (uint32_t)(kXLoads * wave + i)));
#pragma unroll
        for (int i = 0; i < kWLoads; ++i)
            lds_load<4>(wres, live ? woff[i] + (kSK / 2) * (uint32_t)st : kOutOfRange,
                        __builtin_amdgcn_readfirstlane(wb + 256u * (uint32_t)(kWLoads * wave + i)));
        lds_load<2>(sres, live && slane ? soff + (kSK / 32) * (uint32_t)st : kOutOfRange,
                    __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&b.s[wave][0]));
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

#pragma unroll
    for (int st = 0; st < kStages - 1; ++st) issue(st, st);
    for (int s0 = 0; s0 < nsteps; s0 += kStages) {   // unrolled by the stage count: buffer indices are static
#pragma unroll
        for (int p = 0; p < kStages; ++p) {
            const int s = s0 + p;
            if (s >= nsteps) break;   // workgroup-uniform
            wait_vm<kPerStep * (kStages - 2)>();   // this wave's requests of step s are in LDS
            __syncthreads();                        // everyone's are, and step s - 1 is computed
            issue(s + kStages - 1, (p + kStages - 1) % kStages);
            const GemmDmaBuf<kWN, kSK>& b = buf[p];
#pragma unroll
            for (int q = 0; q < kQ; ++q) {
                bf16x8 a[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int row = wn + 32 * i + r32;
                    const uint32_t codes = b.w[row * kWords + ((2 * q + g2) ^ wswz(row))];
                    const int blk = q >> 1;   // the step's 32-column block
                    const uint32_t pair = b.s[row >> 5][(row & 31) + 32 * (blk >> 1)];
                    const float sc = e8m0_scale((pair >> (8 * (blk & 1))) & 0xFFu);
                    const u32x4 u = {fp4x2_to_bf16x2<0>(codes, sc), fp4x2_to_bf16x2<1>(codes, sc),
                                     fp4x2_to_bf16x2<2>(codes, sc), fp4x2_to_bf16x2<3>(codes, sc)};
                    a[i] = __builtin_bit_cast(bf16x8, u);
                }
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int xr = wm + 32 * j + r32;
                    const bf16x8 bx = *reinterpret_cast<const bf16x8*>(&b.x[xr * kSK + 8 * ((2 * q + g2) ^ xswz(xr))]);
#pragma unroll
                    for (int i = 0; i < 2; ++i)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bx, acc[i][j], 0, 0, 0);
                }
            }
        }
    }
    wait_vm<0>();   // the requests past the last step have landed before the workgroup ends

#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int m = m0 + wm + 32 * j + r32;
        if (m >= m_rows) continue;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int nn = n0 + wn + 32 * i + 8 * p + 4 * g2;
                if (nn >= n) continue;
                const int count = min(4, n - nn);
                const f32x4 v = {acc[i][j][4 * p], acc[i][j][4 * p + 1], acc[i][j][4 * p + 2], acc[i][j][4 * p + 3]};
                store4<kBf16Out>(y, (int64_t)m * n + nn, v, count == 4, count);
            }
    }
}

}  // namespace

hipError_t launch_gemm(const uint8_t* packed, const uint8_t* scales, const uint16_t* x, void* y, bool out_bf16,
                       int64_t m, int64_t n, int64_t k, hipStream_t stream) {
    const int ntn = (int)((n + kTileN - 1) / kTileN);
    const int ntm = (int)((m + kTileM - 1) / kTileM);
    const dim3 grid((unsigned)(ntn * ntm));
    if (k % 64 == 0) {
        // weight tiles of 256 rows; with two or more tiles per compute unit, 64-column steps
        // (80 KB of LDS: two workgroups per compute unit), otherwise 128-column steps
        // (fewer barriers per flop; one workgroup per compute unit either way)
        const int ntn4 = (int)((n + 255) / 256);
        const dim3 grid4((unsigned)(ntn4 * ntm));
        const bool wide = k % 128 == 0 && (int64_t)ntn4 * ntm < 2 * (int64_t)device_cu_count();
        const int kc = (int)(k / 32);
        if (wide) {
            if (out_bf16)
                gemm_dma_kernel<true, 3, 4, 128><<<grid4, 512, 0, stream>>>(packed, scales, x, y, (int)m, (int)n, kc);
            else
                gemm_dma_kernel<false, 3, 4, 128><<<grid4, 512, 0, stream>>>(packed, scales, x, y, (int)m, (int)n, kc);
        } else {
            if (out_bf16)
                gemm_dma_kernel<true, 3, 4, 64><<<grid4, 512, 0, stream>>>(packed, scales, x, y, (int)m, (int)n, kc);
            else
                gemm_dma_kernel<false, 3, 4, 64><<<grid4, 512, 0, stream>>>(packed, scales, x, y, (int)m, (int)n, kc);
        }
        return hipGetLastError();
    }
    if (out_bf16)
        gemm_kernel<true><<<grid, kThreads, 0, stream>>>(packed, scales, x, y, (int)m, (int)n, (int)(k / 32));
    else
        gemm_kernel<false><<<grid, kThreads, 0, stream>>>(packed, scales, x, y, (int)m, (int)n, (int)(k / 32));
    return hipGetLastError();
}

}  // namespace e2m1
