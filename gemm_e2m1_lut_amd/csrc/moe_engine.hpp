// moe_engine.hpp -- weight-streaming bf16 MFMA engine of the MoE expert GEMMs:
// an MXFP4 weight matrix read once from HBM against up to 64 bf16 token rows.
//
// Computes acc[t][m] += sum_k W[row of tile t, k] * X[token 16 m + column, k]
// with v_mfma_f32_16x16x32_bf16 (fp32 accumulation) for NT weight tiles of 16
// rows per wave and up to four token tiles of 16 rows per pass.
//
// MFMA lane layout: lane l = 16 g + r holds row r of the A operand (weights)
// and column r of the B operand (tokens), k slots 8 g .. 8 g + 7; D element
// (row 4 g + j, column r) is component j of the accumulator in lane l.
//
// A step is 256 columns, eight E8M0 blocks, one 128-byte line per weight row.
//   * Weights: each wave loads its tiles' lines with coalesced 16-byte loads
//     (one instruction = 8 rows x 128 bytes), two steps ahead of use, and
//     passes them through a private LDS buffer to reach the MFMA layout: lane
//     (r, g) then holds blocks g and g + 4 of row r. The buffer keeps block b
//     of row w at 16-byte slot 8 w + (b ^ (w / 2 % 8)), so the coalesced
//     writes (two rows per 16 lanes) and the MFMA-layout reads (16 rows, one
//     block) have no bank conflicts. Block b = g + 4 h feeds
//     four MFMAs, MFMA i taking codes [8 i, 8 i + 8) of the block as k slots
//     8 g .. 8 g + 7; v_cvt_scalef32_pk_bf16_fp4 decodes two codes and applies
//     the block scale in one instruction.
//   * Scales: the workgroup's rows are 128 consecutive rows of each tile set,
//     so their E8M0 bytes are 128 K / 32 consecutive bytes per set. Where they
//     fit in LDS (NT K / 32 <= 192) the workgroup stages them once per pass
//     with coalesced 16-byte loads, issued before the first weight loads and
//     written before the first product, and every lane reads its block's
//     byte from there. Otherwise (the per-step path) the lane that loads a
//     weight chunk also loads its scale byte, which takes the chunk's LDS
//     route; those scattered byte loads cost about an eighth of the kernel.
//   * Line alignment: a row of K/2 bytes need not start on a 128-byte line
//     (K = 2880: rows start 0, 32, 64 or 96 bytes into a line, repeating every
//     four rows), and a step's 128 bytes of such a row would straddle two
//     lines, each then fetched from HBM by two steps. So a tile takes rows of
//     one line offset 16 mb (stride P, the period of the offsets), and the
//     wave's step s covers the line-aligned columns [256 s - 32 mb, + 256):
//     every weight line is requested by exactly one step. The columns before
//     256 s come from the previous step's token panel (the ring keeps it);
//     the bytes a window reads before a row's start or past its end meet
//     zero tokens, and a resource bounded to the matrix returns zeros for
//     any outside it.
//   * Tokens: the workgroup stages the step's 256 columns of the pass's token
//     rows in a triple-buffered LDS panel, requested two steps ahead and
//     written one step ahead (an L2 round trip per step would otherwise sit
//     in front of every barrier), and every wave reads
//     its B operands from it at the same columns as the A operands, so the
//     column -> k-slot map is the same for both and the sum over k is
//     complete. Columns past K are staged as zeros, so weight blocks past the
//     row end (loaded clamped, finite) add nothing. Panel rows are padded by
//     16 bytes; the B-operand reads of this layout (16 rows per 16 lanes,
//     lane groups 64 bytes apart) run at 0.6 of the LDS's contiguous read
//     rate, but a chunk-major panel that reads at the full rate takes its
//     token loads as 64-byte pieces of 16 rows per wave instead of 512-byte
//     rows, and that measured slower overall.
//
// Every load is issued on every path (indices clamped), the token loads of a
// step before its weight loads, so each wait the compiler places counts
// exactly the loads issued after the one it needs: the weights of step s are
// waited for only when step s is computed, two steps after their request.
#pragma once

#include "device.hpp"

namespace e2m1 {

constexpr int kEngineWaves = 8;
constexpr int kEngineThreads = kEngineWaves * kWave;
constexpr int kEngineStepCols = 256;
constexpr int kEngineMaxTokens = 64;                 // token rows per pass, at most (four MFMA tiles)
constexpr int kPanelPitch = kEngineStepCols + 8;     // bf16 per staged token row (16-byte pad spreads banks)
constexpr int kNonTemporal = 2;                      // cache-policy operand of a buffer load: streaming
constexpr int kStageMaxBlocks = 96;                  // staged path: scale rows of up to 96 blocks (K <= 3072)

template <int N>
struct StaticInt {
    static constexpr int value = N;
};

// Compiler-only fence: keeps loads where they are written (issued early).
// Emits no instruction. The weight and token pointers reaching it are not
// __restrict__: loads through a restrict pointer to read-only memory may be
// moved across.
__device__ __forceinline__ void engine_fence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Rows of K/2 bytes from `base`: the byte offset of row r within its 128-byte
// line repeats with period line_period(K) rows; line_block(base, r, K) is that
// offset in 16-byte blocks (0..7).
__host__ __device__ inline int line_period(int K) {
    int m = (K / 2) & 127, p = 1;
    while ((m * p) & 127) p *= 2;
    return p;
}

__device__ __forceinline__ int line_block(const uint8_t* base, int row, int K) {
    return (int)(((reinterpret_cast<uintptr_t>(base) + (uintptr_t)row * (uintptr_t)(K / 2)) & 127u) >> 4);
}

// Steps that cover K for windows shifted by up to mbmax blocks.
__device__ __forceinline__ int engine_steps(int K, int mbmax) { return (K - 1 + 32 * mbmax) / kEngineStepCols + 1; }

template <int NT>
struct EngineStep {
    uint4 w[NT][2];       // coalesced: rows 8 q + lane / 8 of each tile, block lane % 8
    uint8_t e[NT][2];     // per-step path: E8M0 bytes of the same chunks (bytes: widened at use)
};

// NT 16-row tiles per wave (tile sets of 128 rows per workgroup), passes of
// up to kMaxTok token rows.
template <int NT, int kMaxTok = kEngineMaxTokens>
struct MoeEngine {
    static constexpr int kWBufElems = NT * 16 * 8;   // uint4 per wave: [row][block ^ (row / 2 % 8)]
    static constexpr int kPanelElems = kMaxTok * kPanelPitch;
    static constexpr int kStageBytes = NT * 128 * kStageMaxBlocks;                      // staged E8M0 rows
    static constexpr int kStageChunks = (kStageBytes + kEngineThreads * 16 - 1) / (kEngineThreads * 16);

    // Shared state of one pass (in LDS, owned by the caller's kernel).
    struct Shared {
        uint16_t panel[3][kPanelElems];
        uint4 wbuf[kEngineWaves][kWBufElems];
        union {
            uint8_t sbuf[kEngineWaves][NT * 16 * 8];    // per-step path: E8M0 bytes, [tile][row][block]
            alignas(16) uint8_t stage[kStageBytes];     // staged path: [tile set][128 rows][K / 32]
        };
        int rowidx[kMaxTok];
    };

    // Whether the workgroup's scale rows for reduction length K fit the stage.
    static __host__ __device__ constexpr bool stages(int K) { return NT * 128 * (K / 32) <= kStageBytes; }

    // The scale rows [rb[t], rb[t] + 128) of each tile set t (K / 32 bytes each,
    // 8 K / 32 chunks of 16 bytes per set, read through sres, a resource bounded
    // to the scale matrix: rows past it read zeros): thread i loads chunks i + 512 c.
    static __device__ __forceinline__ void issue_scales(uint4 (&v)[kStageChunks], __amdgpu_buffer_rsrc_t sres,
                                                        int K, const int (&rb)[NT]) {
        const int kb = K / 32, per = 8 * kb;
#pragma unroll
        for (int c = 0; c < kStageChunks; ++c) {
            const int ch = (int)threadIdx.x + kEngineThreads * c;
            int t = 0;   // tile set of the chunk: compares, no division
#pragma unroll
            for (int u = 1; u < NT; ++u) t += ch >= u * per ? 1 : 0;
            // chunks past the stage load offset 0 and are not stored
            const uint32_t off = ch < NT * per ? (uint32_t)(rb[t] * kb + 16 * (ch - t * per)) : 0u;
            const u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(sres, off, 0, kNonTemporal);
            v[c] = make_uint4(u.x, u.y, u.z, u.w);
        }
    }

    static __device__ __forceinline__ void store_scales(const uint4 (&v)[kStageChunks], uint8_t* stage, int K) {
        const int n = NT * 8 * (K / 32);
#pragma unroll
        for (int c = 0; c < kStageChunks; ++c) {
            const int ch = (int)threadIdx.x + kEngineThreads * c;
            if (ch < n) reinterpret_cast<uint4*>(stage)[ch] = v[c];
        }
    }

    // Weight lines (and, on the per-step path, scales) of step `step` for this
    // wave's tiles: tile t is rows row0[t] + stride i (i < 16), clamped to
    // nrows - 1, each starting 16 mb bytes into a 128-byte line; lane l loads 16
    // bytes at 16 (l % 8) of the step's aligned window of row 8 q + l / 8.
    // Scale blocks are clamped to [0, kb - 1] (blocks outside the row meet zero
    // tokens).
    template <bool kStaged>
    static __device__ __forceinline__ void issue_weights(EngineStep<NT>& b, __amdgpu_buffer_rsrc_t wres,
                                                         const uint8_t* ws, int K, const int (&row0)[NT],
                                                         int stride, int mb, int nrows, int step) {
        const int lane = threadIdx.x & (kWave - 1);
        const int kb = K / 32;
        const int blk = 8 * step - mb + (lane & 7);
        const int cb = min(max(blk, 0), kb - 1);
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int row = min(row0[t] + stride * (8 * q + (lane >> 3)), nrows - 1);
                // may lie before the matrix (row 0, step 0): the unsigned offset is then out of
                // range and reads zeros
                const uint32_t off = (uint32_t)(row * (K / 2) + 16 * blk);
                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(wres, off, 0, kNonTemporal);
                b.w[t][q] = make_uint4(v.x, v.y, v.z, v.w);
                if constexpr (!kStaged) b.e[t][q] = ws[(size_t)row * kb + cb];
            }
    }

    // Token columns [256 step, +256) of the pass's first 16 MTA rows: thread t
    // takes 16-byte chunks t + 512 j of the panel (row = chunk / 32), whose
    // source rows src[j] are fixed for the pass.
    template <int MTA>
    static __device__ __forceinline__ void issue_tokens(uint4 (&tr)[MTA], const uint16_t* const (&src)[MTA], int K,
                                                        int step) {
#pragma unroll
        for (int j = 0; j < MTA; ++j) {
            const int ch = ((int)threadIdx.x + kEngineThreads * j) & 31;
            const int col = min(step * kEngineStepCols + 8 * ch, K - 8);
            tr[j] = *reinterpret_cast<const uint4*>(src[j] + col);
        }
    }

    template <int MTA>
    static __device__ __forceinline__ void store_tokens(const uint4 (&tr)[MTA], uint16_t* panel, int K, int step) {
#pragma unroll
        for (int j = 0; j < MTA; ++j) {
            const int id = (int)threadIdx.x + kEngineThreads * j;
            const int row = id >> 5, ch = id & 31;
            // columns past K stage as zeros (a mask, not a select: a select lets the
            // compiler turn the load into a conditional one placed after the weights)
            const uint32_t keep = step * kEngineStepCols + 8 * ch < K ? ~0u : 0u;
            *reinterpret_cast<uint4*>(panel + row * kPanelPitch + 8 * ch) =
                make_uint4(tr[j].x & keep, tr[j].y & keep, tr[j].z & keep, tr[j].w & keep);
        }
    }

    // acc += step s held in b (weights) x token panels. The wave's columns are
    // [256 s - 32 mb, + 256): those before 256 s are read from the previous
    // step's panel (zero at the first step). Staged scales: lane (r, g) reads
    // stage[soff[t] + block], soff[t] the start of its row of tile t.
    template <int MTA, bool kStaged>
    static __device__ __forceinline__ void compute(const EngineStep<NT>& b, uint4* wbuf, uint8_t* sbuf,
                                                   const uint8_t* stage, const int (&soff)[NT], int K, int s,
                                                   const uint16_t* panel, const uint16_t* prev, int mb,
                                                   f32x4 (&acc)[NT][4]) {
        const int lane = threadIdx.x & (kWave - 1);
        const int r = lane & 15, g = lane >> 4;
        const bool first = s == 0;
        // coalesced lines (and their scale bytes) -> MFMA layout through the wave's LDS buffers
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int row = t * 16 + 8 * q + (lane >> 3);
                wbuf[row * 8 + ((lane & 7) ^ ((row >> 1) & 7))] = b.w[t][q];
                if constexpr (!kStaged) sbuf[row * 8 + (lane & 7)] = b.e[t][q];
            }
        uint4 a4[NT][2];
        uint32_t e4[NT][2];
        const int blk = 8 * s - mb + g;   // this lane's first block of the step (g + 4 h: the second)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                a4[t][h] = wbuf[(t * 16 + r) * 8 + ((g + 4 * h) ^ ((r >> 1) & 7))];
                if constexpr (kStaged)
                    e4[t][h] = stage[soff[t] + min(max(blk + 4 * h, 0), K / 32 - 1)];
                else
                    e4[t][h] = sbuf[(t * 16 + r) * 8 + g + 4 * h];
            }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            float sc[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) sc[t] = e8m0_scale(e4[t][h]);
            // this lane's token columns for block g + 4 h, relative to the step's panel
            const int cb = 32 * (g + 4 * h - mb);
            const bool from_prev = cb < 0;
            const uint16_t* src = (from_prev ? prev : panel) + r * kPanelPitch + (from_prev ? cb + 256 : cb);
            const bool zero = first && from_prev;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bf16x8 a[NT];
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const uint32_t wd = i == 0 ? a4[t][h].x : i == 1 ? a4[t][h].y : i == 2 ? a4[t][h].z : a4[t][h].w;
                    const u32x4 u = {fp4x2_to_bf16x2<0>(wd, sc[t]), fp4x2_to_bf16x2<1>(wd, sc[t]),
                                     fp4x2_to_bf16x2<2>(wd, sc[t]), fp4x2_to_bf16x2<3>(wd, sc[t])};
                    a[t] = __builtin_bit_cast(bf16x8, u);
                }
#pragma unroll
                for (int m = 0; m < MTA; ++m) {
                    u32x4 xw = *reinterpret_cast<const u32x4*>(src + 16 * m * kPanelPitch + 8 * i);
                    if (zero) xw = u32x4{0u, 0u, 0u, 0u};
                    const bf16x8 bx = __builtin_bit_cast(bf16x8, xw);
#pragma unroll
                    for (int t = 0; t < NT; ++t)
                        acc[t][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[t], bx, acc[t][m], 0, 0, 0);
                }
            }
        }
    }

    // The whole product over K for one pass of MTA token tiles. sh.rowidx
    // holds the pass's source rows (written and synchronised by the caller);
    // nsteps covers the latest window of the workgroup's waves. Staged path:
    // rb[t] is the first of the workgroup's 128 rows of tile set t (row0[t] +
    // stride i lies in [rb[t], rb[t] + 128)), sres the scale matrix's resource.
    template <int MTA, bool kStaged>
    static __device__ __forceinline__ void run(Shared& sh, __amdgpu_buffer_rsrc_t wres, const uint8_t* ws,
                                               __amdgpu_buffer_rsrc_t sres, const int (&rb)[NT], int K,
                                               const int (&row0)[NT], int stride, int mb, int nsteps, int nrows,
                                               const uint16_t* xb, size_t xpitch, int nvalid, f32x4 (&acc)[NT][4]) {
        const int wave = threadIdx.x / kWave;
        uint4* wbuf = sh.wbuf[wave];
        uint8_t* sbuf = sh.sbuf[wave];
        const uint16_t* src[MTA];
#pragma unroll
        for (int j = 0; j < MTA; ++j) {
            const int row = ((int)threadIdx.x + kEngineThreads * j) >> 5;
            src[j] = xb + (size_t)sh.rowidx[min(row, nvalid - 1)] * xpitch;
        }
        int soff[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) soff[t] = (128 * t + row0[t] - rb[t] + stride * (int)(threadIdx.x & 15)) * (K / 32);
        uint4 pre[kStageChunks];
        // first, so that the wait before their LDS store counts the step loads issued after them
        if constexpr (kStaged) issue_scales(pre, sres, K, rb);
        EngineStep<NT> buf[3];
        uint4 tr[2][MTA];
        // Sub-iteration s (from -2): requests the weights and tokens of step s + 2
        // (weights into buffer (s + 2) % 3, tokens into registers s % 2), computes
        // step s from buffer s % 3 and panel s % 3 (panel (s - 1) % 3 still holds
        // step s - 1), then writes the tokens of step s + 1 (requested one
        // sub-iteration ago) to panel (s + 1) % 3. B = (s + 2) % 6 makes every
        // buffer index static; the first two sub-iterations only issue loads.
        auto sub = [&](auto bc, int s) __attribute__((always_inline)) {
            constexpr int B = decltype(bc)::value;
            const int next = min(s + 2, nsteps - 1);
            issue_tokens<MTA>(tr[B & 1], src, K, next);
            engine_fence();
            issue_weights<kStaged>(buf[B % 3], wres, ws, K, row0, stride, mb, nrows, next);
            engine_fence();
            if (s >= 0)
                compute<MTA, kStaged>(buf[(B + 1) % 3], wbuf, sbuf, sh.stage, soff, K, s, sh.panel[(B + 1) % 3],
                                      sh.panel[B % 3], mb, acc);
            engine_fence();
            if (s + 1 >= 0) store_tokens<MTA>(tr[(B + 1) & 1], sh.panel[(B + 2) % 3], K, min(s + 1, nsteps - 1));
            __syncthreads();
        };
        // (a peeled prologue makes the compiler spill: the loop form keeps the
        // buffers in registers)
        for (int it = -2; it < nsteps; it += 6) {   // exits are workgroup-uniform
            sub(StaticInt<0>{}, it);
            if (it + 1 >= nsteps) break;
            sub(StaticInt<1>{}, it + 1);
            if constexpr (kStaged) {
                if (it == -2) {   // the staged scales are in LDS before step 0 is computed
                    store_scales(pre, sh.stage, K);
                    __syncthreads();
                }
            }
            if (it + 2 >= nsteps) break;
            sub(StaticInt<2>{}, it + 2);
            if (it + 3 >= nsteps) break;
            sub(StaticInt<3>{}, it + 3);
            if (it + 4 >= nsteps) break;
            sub(StaticInt<4>{}, it + 4);
            if (it + 5 >= nsteps) break;
            sub(StaticInt<5>{}, it + 5);
        }
    }

    // run<MTA> for MTA = mt (1 <= mt <= 4), chosen once per pass.
    template <bool kStaged>
    static __device__ __forceinline__ void run_mt(int mt, Shared& sh, __amdgpu_buffer_rsrc_t wres, const uint8_t* ws,
                                                  __amdgpu_buffer_rsrc_t sres, const int (&rb)[NT], int K,
                                                  const int (&row0)[NT], int stride, int mb, int nsteps, int nrows,
                                                  const uint16_t* xb, size_t xpitch, int nvalid, f32x4 (&acc)[NT][4]) {
        constexpr int kTop = kMaxTok / 16;
        switch (mt) {
            case 1: run<1, kStaged>(sh, wres, ws, sres, rb, K, row0, stride, mb, nsteps, nrows, xb, xpitch, nvalid, acc); break;
            case 2: run<2, kStaged>(sh, wres, ws, sres, rb, K, row0, stride, mb, nsteps, nrows, xb, xpitch, nvalid, acc); break;
            case 3: run<(kTop < 3 ? kTop : 3), kStaged>(sh, wres, ws, sres, rb, K, row0, stride, mb, nsteps, nrows, xb, xpitch, nvalid, acc); break;
            default: run<kTop, kStaged>(sh, wres, ws, sres, rb, K, row0, stride, mb, nsteps, nrows, xb, xpitch, nvalid, acc); break;
        }
    }
};

}  // namespace e2m1
