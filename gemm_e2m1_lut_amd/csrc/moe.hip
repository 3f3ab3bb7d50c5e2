// moe.hip -- MXFP4 mixture-of-experts layer (mxfp4_moe_gemm).
//
// Semantics: the fused expert op exercised by the MoE test of the vLLM pull
// request 51583 digest (section "关键源码片段"): the first expert matrix W13
// has 2 * inter rows (gate rows first, then up rows), the activation is
// silu(gate) * up, the second matrix W2 maps back to hidden, and each token's
// top-k slot outputs are weighted by the routing weights and summed. Routing
// (ids and weights) is an input. Weights are MXFP4 with the unpack of the same
// page ("功能与动机": E2M1 lookup, E8M0 block scale as an exponent add).
//
// gfx950 design (four launches on the caller's stream):
//   1. route: one workgroup turns topk_ids into per-expert counts, offsets
//      and a stable (token, slot)-ordered list of rows per expert, using
//      wave ballots for the ranks (no atomics, so the layout is deterministic).
//   2. gemm1: a workgroup of eight waves owns one expert and 128 intermediate
//      columns j: wave w streams the gate rows j0 + 16 w .. + 15 and the
//      matching up rows of W13 through the engine of moe_engine.hpp against
//      the expert's token rows (up to 64 per pass), so every weight byte is
//      read once for all tokens of its expert; the epilogue applies
//      silu(gate) * up in fp32 and stores the activation as bf16 (the MFMA
//      operand type of gemm2).
//   3. gemm2: the same engine over W2, three 16-row tiles per wave (rows h,
//      h + 128 and h + 256), 384 hidden rows per workgroup and passes of up to
//      48 activation rows, with the activations as operand; fp32 results per
//      (expert row, hidden). Several tiles per wave divide the token panel
//      bytes staged per weight byte, and with three the 2880-row layer's
//      8 x 32 workgroups fill 256 compute units once (one tile: 58.5 us for
//      the 32-expert 2880 x 2880 layer, two: 52.4 us, three: 44.0 us).
//   4. combine: out[t] = bf16(sum over slots, in slot order, of weight * y).
//   Lane layout of the MFMA (checked on the device): lane l holds row l % 16
//   of A and column l % 16 of B, k = 8 * (l / 16) + 0..7; D row 4 * (l / 16) +
//   0..3, column l % 16. A lane's 16-byte weight chunk is one 32-column scale
//   block; over four MFMAs its 32 codes cover the k slots of its lane group,
//   and the token rows are read from LDS with the same k order.
#include "device.hpp"
#include "kernels.hpp"
#include "moe_engine.hpp"

namespace e2m1 {
namespace {

constexpr int kMaxExperts = 512;
constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / kWave;

constexpr int kThreads = kEngineThreads;             // 8 waves
constexpr int kGemm1Cols = kEngineWaves * 16;         // 128 intermediate columns per block (gate + up tiles)
constexpr int kG2Tiles = 3;                           // gemm2: 16-row tiles per wave
constexpr int kG2Tokens = 48;                         // gemm2: activation rows per pass
constexpr int kGemm2Rows = kEngineWaves * 16 * kG2Tiles;   // 384 hidden rows per block

struct MoeLayout {
    size_t cnt, off, pair_row, row_pair, act, y, total;
};

__host__ __device__ inline MoeLayout moe_layout(int64_t tokens, int64_t hidden, int64_t inter,
                                               int64_t experts, int64_t topk) {
    auto a = [](size_t v) { return (v + 255) & ~(size_t)255; };
    const size_t P = (size_t)(tokens * topk);
    MoeLayout L;
    L.cnt = 0;
    L.off = L.cnt + a(4 * (size_t)experts);
    L.pair_row = L.off + a(4 * (size_t)(experts + 1));
    L.row_pair = L.pair_row + a(4 * P);
    L.act = L.row_pair + a(4 * P);
    L.y = L.act + a(2 * P * (size_t)inter);
    L.total = L.y + a(4 * P * (size_t)hidden);
    return L;
}

// ------------------------------------------------------------------ route --

constexpr int kRouteKeep = 4;   // chunks of kRouteThreads pairs whose ranks stay in registers

// One workgroup. Pairs are taken in chunks of kRouteThreads (pair p0 + t by
// thread t). Within a chunk a pair's rank among the pairs of its wave with the
// same expert comes from wave ballots (lanes in order); the per-wave counts
// become per-wave bases with a prefix over the waves (in wave order, after
// the pairs of earlier chunks), so a pair's row within its expert is base +
// rank: the order is (token, slot) order and needs no atomics. Rows of the
// first kRouteKeep chunks stay in registers until the experts' offsets are
// known; later chunks park them in pair_row. The offsets are an exclusive
// prefix over the experts (waves of 64 experts, then the wave totals).
__global__ __launch_bounds__(kRouteThreads) void moe_route_kernel(const int32_t* __restrict__ ids,
                                                                  int P, int E, int* __restrict__ cnt,
                                                                  int* __restrict__ off,
                                                                  int* __restrict__ pair_row,
                                                                  int* __restrict__ row_pair) {
    __shared__ int s_wave[kRouteWaves][kMaxExperts];   // per-wave counts, then wave bases
    __shared__ int s_count[kMaxExperts];               // pairs per expert so far
    __shared__ int s_off[kMaxExperts];                 // first row of each expert
    __shared__ int s_wtot[kRouteWaves];                // pairs of each wave's 64 experts
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    for (int x = tid; x < E; x += kRouteThreads) s_count[x] = 0;
    // pair p0 + tid: its expert (-1 if none or out of range) and its row within the expert
    auto chunk = [&](int p0, int& e_out, int& row_out) __attribute__((always_inline)) {
        for (int i = tid; i < kRouteWaves * E; i += kRouteThreads) s_wave[i / E][i % E] = 0;
        __syncthreads();
        const int p = p0 + tid;
        int e = (p < P) ? ids[p] : -1;
        if (e < 0 || e >= E) e = -1;
        int rank = 0;
        uint64_t pending = __ballot(e >= 0);
        while (pending) {
            const int leader = __ffsll((unsigned long long)pending) - 1;
            const int X = __builtin_amdgcn_readlane(e, leader);   // leader is wave-uniform: no LDS round trip
            const uint64_t m = __ballot(e == X);
            if (e == X) rank = __popcll(m & lower);
            if (lane == leader) s_wave[wave][X] = __popcll(m);
            pending &= ~m;
        }
        __syncthreads();
        for (int x = tid; x < E; x += kRouteThreads) {   // wave bases of expert x, continuing s_count
            int c[kRouteWaves];
#pragma unroll
            for (int w = 0; w < kRouteWaves; ++w) c[w] = s_wave[w][x];
            int run = s_count[x];
#pragma unroll
            for (int w = 0; w < kRouteWaves; ++w) {
                s_wave[w][x] = run;
                run += c[w];
            }
            s_count[x] = run;
        }
        __syncthreads();
        e_out = e;
        row_out = e >= 0 ? s_wave[wave][e] + rank : 0;
        __syncthreads();   // s_wave is cleared by the next chunk
    };
    int keep_e[kRouteKeep], keep_r[kRouteKeep];
#pragma unroll
    for (int c = 0; c < kRouteKeep; ++c) {
        keep_e[c] = -1;
        keep_r[c] = 0;
        if (c * kRouteThreads < P) chunk(c * kRouteThreads, keep_e[c], keep_r[c]);   // workgroup-uniform
    }
    for (int p0 = kRouteKeep * kRouteThreads; p0 < P; p0 += kRouteThreads) {
        int e, r;
        chunk(p0, e, r);
        if (p0 + tid < P) pair_row[p0 + tid] = e >= 0 ? r : -1;
    }
    // exclusive prefix of the counts over the experts: expert x = 64 wave + lane
    {
        const int x = tid;
        const int v = x < E ? s_count[x] : 0;
        int incl = v;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int u = __shfl_up(incl, d, kWave);
            if (lane >= d) incl += u;
        }
        if (lane == kWave - 1) s_wtot[wave] = incl;
        __syncthreads();
        int base = 0;
        for (int w = 0; w < wave; ++w) base += s_wtot[w];   // wave-uniform
        if (x < E) {
            s_off[x] = base + incl - v;
            cnt[x] = v;
            off[x] = base + incl - v;
        }
        if (x == E - 1) off[E] = base + incl;
        __syncthreads();
    }
#pragma unroll
    for (int c = 0; c < kRouteKeep; ++c) {
        const int p = c * kRouteThreads + tid;
        if (p < P) {
            const int e = keep_e[c];
            if (e >= 0) {
                const int r = s_off[e] + keep_r[c];
                pair_row[p] = r;
                row_pair[r] = p;
            } else {
                pair_row[p] = -1;
            }
        }
    }
    for (int p = kRouteKeep * kRouteThreads + tid; p < P; p += kRouteThreads) {
        const int r0 = pair_row[p];
        if (r0 >= 0) {
            const int r = s_off[ids[p]] + r0;
            pair_row[p] = r;
            row_pair[r] = p;
        }
    }
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + __expf(-z)); }

// Workgroups go to the eight XCDs round-robin by launch index, and each XCD
// has its own L2. The launch index is remapped so that XCD x gets the
// contiguous range [x * per, (x + 1) * per) of (expert, block) work items in
// expert-major order: the token or activation rows of an expert are then read
// into one L2 only (the activations of all experts are larger than one L2).
constexpr int kXcds = 8;

struct MoeWork {
    int e, blk;
    bool valid;
};

__device__ __forceinline__ MoeWork moe_work(int blocks_per_expert, int experts) {
    const int total = blocks_per_expert * experts;
    const int per = (total + kXcds - 1) / kXcds;
    const int w = (int)(blockIdx.x % kXcds) * per + (int)(blockIdx.x / kXcds);
    MoeWork m;
    m.valid = w < total;
    m.e = m.valid ? w / blocks_per_expert : 0;
    m.blk = m.valid ? w % blocks_per_expert : 0;
    return m;
}

inline int moe_grid(int blocks_per_expert, int experts) {
    const int total = blocks_per_expert * experts;
    return kXcds * ((total + kXcds - 1) / kXcds);
}

// ----------------------------------------------------------------- gemm1 --

using Gemm1 = MoeEngine<2>;
using Gemm2 = MoeEngine<kG2Tiles, kG2Tokens>;
static_assert(sizeof(Gemm2::Shared::panel) >= kG2Tokens * (kGemm2Rows + 4) * sizeof(float), "gemm2 staging");

// Workgroup (j block, expert): wave w streams gate rows j0 + 16 w .. + 15 and
// up rows inter + the same j against all of the expert's tokens (64 per pass),
// then act = silu(gate) * up. kStaged: the block's scale rows are staged in LDS.
template <bool kStaged>
__global__ __launch_bounds__(kThreads) void moe_gemm1_kernel(
    const uint16_t* x, const uint8_t* w13, const uint8_t* w13s,
    const int* __restrict__ cnt, const int* __restrict__ off, const int* __restrict__ row_pair,
    uint16_t* __restrict__ act, int H, int I, int E, int topk) {
    __shared__ Gemm1::Shared sh;
    const MoeWork work = moe_work((I + kGemm1Cols - 1) / kGemm1Cols, E);
    if (!work.valid) return;
    const int e = work.e;
    const int n_e = cnt[e];
    if (n_e == 0) return;
    const int base = off[e];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // wave-uniform
    const int g = lane >> 4, r16 = lane & 15;
    const uint8_t* we = w13 + (size_t)e * 2 * I * (H / 2);
    const uint8_t* se = w13s + (size_t)e * 2 * I * (H / 32);
    // rows of one line offset per tile: wave w takes j = j0 + P (4 g' + jj) + c for its 16
    // columns j (c = w % P, 16 P consecutive j per group of P waves), gate rows j and up rows I + j
    // (I (H / 2) is a multiple of 128: the same offsets)
    const int P = line_period(H);
    const int jb = work.blk * kGemm1Cols;
    const int j0 = jb + 16 * P * (wave / P) + wave % P;
    const int row0[2] = {j0, I + j0};
    const int rb[2] = {jb, I + jb};
    const int mb = line_block(we, j0, H);
    int mbmax = 0;
    for (int c = 0; c < P; ++c) mbmax = max(mbmax, line_block(we, work.blk * kGemm1Cols + c, H));
    const int nsteps = engine_steps(H, mbmax);
    const __amdgpu_buffer_rsrc_t wres =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(we), 0, 2 * I * (H / 2), kBufferWord3);
    const __amdgpu_buffer_rsrc_t sres =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(se), 0, 2 * I * (H / 32), kBufferWord3);

    for (int m0 = 0; m0 < n_e; m0 += kEngineMaxTokens) {
        const int nv = min(kEngineMaxTokens, n_e - m0);
        const int mt = (nv + 15) / 16;
        __syncthreads();   // the previous pass is done with rowidx and the panels
        if ((int)threadIdx.x < nv) sh.rowidx[threadIdx.x] = row_pair[base + m0 + threadIdx.x] / topk;
        __syncthreads();
        f32x4 acc[2][4];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int m = 0; m < 4; ++m) acc[t][m] = f32x4{0.f, 0.f, 0.f, 0.f};
        Gemm1::run_mt<kStaged>(mt, sh, wres, se, sres, rb, H, row0, P, mb, nsteps, 2 * I, x, (size_t)H, nv, acc);
        // epilogue: act = silu(gate) * up -> bf16; lane (g, r) holds j = j0 + P (4 g + jj), jj < 4.
        // With P > 1 the workgroup's 128 j of each token row are interleaved over its waves, so
        // they meet in LDS (over the token panels, free once every wave is past the product) and
        // leave as contiguous 16-byte stores.
        if (P == 1) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int r = 16 * m + r16;
                const int j = j0 + 4 * g;
                if (m < mt && r < nv && j < I) {
                    const f32x4 gt = acc[0][m], up = acc[1][m];
                    const uint32_t lo = pack_bf16x2(silu_f32(gt[0]) * up[0], silu_f32(gt[1]) * up[1]);
                    const uint32_t hi = pack_bf16x2(silu_f32(gt[2]) * up[2], silu_f32(gt[3]) * up[3]);
                    *reinterpret_cast<uint2*>(act + (size_t)(base + m0 + r) * I + j) = make_uint2(lo, hi);
                }
            }
        } else {
            uint16_t* stage = &sh.panel[0][0];   // [64 tokens][kGemm1Cols + 8]
            constexpr int kStagePitch = kGemm1Cols + 8;
            __syncthreads();   // every wave is done with the panels
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int r = 16 * m + r16;
                if (m < mt && r < nv) {
                    const f32x4 gt = acc[0][m], up = acc[1][m];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        stage[r * kStagePitch + (j0 - jb) + P * (4 * g + jj)] =
                            (uint16_t)f32_to_bf16_rne(silu_f32(gt[jj]) * up[jj]);
                }
            }
            __syncthreads();
            for (int i = threadIdx.x; i < nv * (kGemm1Cols / 8); i += kThreads) {
                const int r = i / (kGemm1Cols / 8), c8 = 8 * (i % (kGemm1Cols / 8));
                if (jb + c8 < I)
                    *reinterpret_cast<uint4*>(act + (size_t)(base + m0 + r) * I + jb + c8) =
                        *reinterpret_cast<const uint4*>(stage + r * kStagePitch + c8);
            }
        }
    }
}

// ----------------------------------------------------------------- gemm2 --

// Workgroup (hidden block, expert): wave w streams the W2 rows of its three
// tiles (h0 + 128 t + P i, t < 3, i < 16) against the expert's activation
// rows; fp32 results per (expert row, hidden).
template <bool kStaged>
__global__ __launch_bounds__(kThreads) void moe_gemm2_kernel(
    const uint16_t* act, const uint8_t* w2, const uint8_t* w2s,
    const int* __restrict__ cnt, const int* __restrict__ off, float* __restrict__ y, int H, int I, int E) {
    __shared__ Gemm2::Shared sh;
    const MoeWork work = moe_work((H + kGemm2Rows - 1) / kGemm2Rows, E);
    if (!work.valid) return;
    const int e = work.e;
    const int n_e = cnt[e];
    if (n_e == 0) return;
    const int base = off[e];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // wave-uniform
    const int g = lane >> 4, r16 = lane & 15;
    const uint8_t* we = w2 + (size_t)e * H * (I / 2);
    const uint8_t* se = w2s + (size_t)e * H * (I / 32);
    // rows of one line offset per tile, as in gemm1: h = h0 + P (4 g' + jj) + c
    const int P = line_period(I);
    const int hb = work.blk * kGemm2Rows;
    const int h0 = hb + 16 * P * (wave / P) + wave % P;
    int row0[kG2Tiles], rb[kG2Tiles];   // tiles 128 rows apart: rows of I / 2 bytes keep their line offsets
#pragma unroll
    for (int t = 0; t < kG2Tiles; ++t) {
        row0[t] = h0 + 128 * t;
        rb[t] = hb + 128 * t;
    }
    const int mb = line_block(we, h0, I);
    int mbmax = 0;
    for (int c = 0; c < P; ++c) mbmax = max(mbmax, line_block(we, work.blk * kGemm2Rows + c, I));
    const int nsteps = engine_steps(I, mbmax);
    const __amdgpu_buffer_rsrc_t wres =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(we), 0, H * (I / 2), kBufferWord3);
    const __amdgpu_buffer_rsrc_t sres =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(se), 0, H * (I / 32), kBufferWord3);

    for (int m0 = 0; m0 < n_e; m0 += kG2Tokens) {
        const int nv = min(kG2Tokens, n_e - m0);
        const int mt = (nv + 15) / 16;
        __syncthreads();
        if ((int)threadIdx.x < nv) sh.rowidx[threadIdx.x] = base + m0 + threadIdx.x;
        __syncthreads();
        f32x4 acc[kG2Tiles][4];
#pragma unroll
        for (int t = 0; t < kG2Tiles; ++t)
#pragma unroll
            for (int m = 0; m < 4; ++m) acc[t][m] = f32x4{0.f, 0.f, 0.f, 0.f};
        Gemm2::run_mt<kStaged>(mt, sh, wres, se, sres, rb, I, row0, P, mb, nsteps, H, act, (size_t)I, nv, acc);
        // lane (g, r) holds h = h0 + P (4 g + jj), jj < 4: with P > 1 the workgroup's 128 h of each
        // token row are interleaved over its waves, so they meet in LDS (over the token panels, free
        // once every wave is past the product) and leave as contiguous 16-byte stores
        if (P == 1) {
#pragma unroll
            for (int t = 0; t < kG2Tiles; ++t)
#pragma unroll
                for (int m = 0; m < kG2Tokens / 16; ++m) {
                    const int r = 16 * m + r16;
                    const int h = h0 + 128 * t + 4 * g;
                    if (m < mt && r < nv && h + 3 < H)
                        *reinterpret_cast<f32x4*>(y + (size_t)(base + m0 + r) * H + h) = acc[t][m];
                }
        } else {
            float* stage = reinterpret_cast<float*>(&sh.panel[0][0]);   // [48 tokens][kGemm2Rows + 4]
            constexpr int kStagePitch = kGemm2Rows + 4;
            __syncthreads();   // every wave is done with the panels
#pragma unroll
            for (int t = 0; t < kG2Tiles; ++t)
#pragma unroll
                for (int m = 0; m < kG2Tokens / 16; ++m) {
                    const int r = 16 * m + r16;
                    if (m < mt && r < nv) {
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj)
                            stage[r * kStagePitch + (h0 - hb) + 128 * t + P * (4 * g + jj)] = acc[t][m][jj];
                    }
                }
            __syncthreads();
            for (int i = threadIdx.x; i < nv * (kGemm2Rows / 4); i += kThreads) {
                const int r = i / (kGemm2Rows / 4), c4 = 4 * (i % (kGemm2Rows / 4));
                if (hb + c4 + 3 < H)
                    *reinterpret_cast<f32x4*>(y + (size_t)(base + m0 + r) * H + hb + c4) =
                        *reinterpret_cast<const f32x4*>(stage + r * kStagePitch + c4);
            }
        }
    }
}

// --------------------------------------------------------------- combine --

constexpr int kCombineThreads = 256;   // 256-thread workgroups: the 256-token layer fills every compute unit

// out[t] = bf16(sum over slots j, in slot order, of weights[t, j] * y[row of (t, j)]):
// thread i takes token i / (H / 8), columns 8 (i % (H / 8)) .. + 7. The rows and
// weights of four slots are read first, then their eight 16-byte y loads, so
// the slots' latencies overlap; a slot without a row (an expert id outside the
// range) reads row 0 and adds nothing.
__global__ __launch_bounds__(kCombineThreads) void moe_combine_kernel(const float* __restrict__ y,
                                                                      const int* __restrict__ pair_row,
                                                                      const float* __restrict__ weights,
                                                                      uint16_t* __restrict__ out, int T, int H,
                                                                      int topk) {
    const int chunks = H / 8;
    const int64_t total = (int64_t)T * chunks;
    for (int64_t i = (int64_t)blockIdx.x * kCombineThreads + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * kCombineThreads) {
        const int t = (int)(i / chunks);
        const int c = (int)(i % chunks);
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int j0 = 0; j0 < topk; j0 += 4) {
            int r[4];
            float w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int j = min(j0 + q, topk - 1);
                r[q] = j0 + q < topk ? pair_row[t * topk + j] : -1;
                w[q] = weights[t * topk + j];
            }
            f32x4 v[4][2];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4* src = reinterpret_cast<const f32x4*>(y + (size_t)max(r[q], 0) * H + 8 * c);
                v[q][0] = src[0];
                v[q][1] = src[1];
            }
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (r[q] >= 0) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc[e] += w[q] * v[q][0][e];
                        acc[4 + e] += w[q] * v[q][1][e];
                    }
                }
        }
        uint4 o;
        o.x = pack_bf16x2(acc[0], acc[1]);
        o.y = pack_bf16x2(acc[2], acc[3]);
        o.z = pack_bf16x2(acc[4], acc[5]);
        o.w = pack_bf16x2(acc[6], acc[7]);
        *reinterpret_cast<uint4*>(out + (size_t)t * H + 8 * c) = o;
    }
}

}  // namespace

size_t moe_workspace_bytes(int64_t tokens, int64_t hidden, int64_t inter, int64_t experts,
                           int64_t topk) {
    return moe_layout(tokens, hidden, inter, experts, topk).total;
}

hipError_t launch_moe(const uint16_t* x, const uint8_t* w13, const uint8_t* w13s,
                      const uint8_t* w2, const uint8_t* w2s, const int32_t* ids,
                      const float* weights, uint16_t* out, void* workspace, int64_t tokens,
                      int64_t hidden, int64_t inter, int64_t experts, int64_t topk,
                      hipStream_t stream) {
    if (experts > kMaxExperts) return hipErrorInvalidValue;
    const MoeLayout L = moe_layout(tokens, hidden, inter, experts, topk);
    uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
    int* cnt = reinterpret_cast<int*>(ws + L.cnt);
    int* off = reinterpret_cast<int*>(ws + L.off);
    int* pair_row = reinterpret_cast<int*>(ws + L.pair_row);
    int* row_pair = reinterpret_cast<int*>(ws + L.row_pair);
    uint16_t* act = reinterpret_cast<uint16_t*>(ws + L.act);
    float* y = reinterpret_cast<float*>(ws + L.y);
    const int P = (int)(tokens * topk), E = (int)experts, H = (int)hidden, I = (int)inter;

    moe_route_kernel<<<1, kRouteThreads, 0, stream>>>(ids, P, E, cnt, off, pair_row, row_pair);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // scale rows are staged in LDS where they fit and start 16-byte aligned (every
    // workgroup's rows then do: 128 rows of K / 32 bytes are a multiple of 16)
    auto aligned16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    const int g1 = moe_grid((I + kGemm1Cols - 1) / kGemm1Cols, E);
    if (Gemm1::stages(H) && aligned16(w13s))
        moe_gemm1_kernel<true><<<g1, kThreads, 0, stream>>>(x, w13, w13s, cnt, off, row_pair, act, H, I, E, (int)topk);
    else
        moe_gemm1_kernel<false><<<g1, kThreads, 0, stream>>>(x, w13, w13s, cnt, off, row_pair, act, H, I, E, (int)topk);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const int g2 = moe_grid((H + kGemm2Rows - 1) / kGemm2Rows, E);
    if (Gemm2::stages(I) && aligned16(w2s))
        moe_gemm2_kernel<true><<<g2, kThreads, 0, stream>>>(act, w2, w2s, cnt, off, y, H, I, E);
    else
        moe_gemm2_kernel<false><<<g2, kThreads, 0, stream>>>(act, w2, w2s, cnt, off, y, H, I, E);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const int64_t chunks = tokens * (hidden / 8);
    const int64_t want = (chunks + kCombineThreads - 1) / kCombineThreads;
    const int grid = (int)(want < 8192 ? want : 8192);
    moe_combine_kernel<<<grid, kCombineThreads, 0, stream>>>(y, pair_row, weights, out, (int)tokens, H, (int)topk);
    return hipGetLastError();
}

}  // namespace e2m1
