// mfma_panel.hpp -- streamed-weight bf16 MFMA engine: an MXFP4 weight matrix
// read once from HBM against a few bf16 token rows staged in LDS.
//
// Computes acc[t][m] += sum_k W[row of tile t, k] * X[token row of tile m, k]
// with v_mfma_f32_16x16x32_bf16 (fp32 accumulation) for NT weight tiles of 16
// rows per wave and up to MT token tiles of 16 rows per block.
//
// Lane layout (one wave): lane l = 16 g + r belongs to row r of every operand
// tile and to lane group g. A step covers 256 columns = 8 scale blocks = one
// 128-byte line of codes per weight row: lane (r, g) loads the 16 bytes of
// blocks g and g + 4 of its row (the two halves of the line are requested
// back to back) and their two E8M0 bytes. Block b = g + 4 h feeds four MFMAs,
// MFMA i taking codes [8 i, 8 i + 8) of the block as the lane's A operand
// (MFMA k slot 8 g + 0..7); the token operand of the same MFMA is read from
// LDS at the same columns, so both operands share one column -> k-slot map and
// the sum over k is complete. v_cvt_scalef32_pk_bf16_fp4 decodes two codes and
// applies the block scale in one instruction. D element (row 4 g + j, column
// r) of tile (t, m) is component j of acc[t][m] in lane l: weight row
// 16 t + 4 g + j, token 16 m + r.
//
// Token rows are staged in LDS panels of 512 columns, double-buffered: while
// panel p is multiplied, every thread already holds its share of panel p + 1
// in registers (loaded before the weights of the panel's second step), and
// writes it to the other buffer at the end of the panel, followed by the one
// barrier per panel. Weights are loaded into two step buffers, the next step's
// loads issued as soon as a buffer is consumed. Because vector-memory loads
// complete in issue order, every wait in this order is for loads issued at
// least one step earlier: no wait ever stalls on a load just issued.
//
// Loads are unconditional with indices clamped into range and masked at use
// (a load under a condition makes the compiler wait for it before the
// alternative value is written). Columns past K read finite data (clamped)
// and meet zero codes; token rows past the valid count hold data that only
// reaches D columns which are never stored.
#pragma once

#include "device.hpp"

namespace e2m1 {

constexpr int kStepCols = 256;
constexpr int kPanelCols = 512;
constexpr int kPanelPitch = kPanelCols + 8;   // bf16 per staged row: 16-byte pad spreads LDS banks

struct WeightStep {
    uint4 w[2];          // codes of blocks g and g + 4 of the step
    uint32_t e[2];       // their E8M0 bytes
};

// A compiler-only fence: memory operations are not moved across it, so loads
// stay where they are written (issued early) instead of being sunk next to the
// loop-carried uses in the next iteration. Emits no instruction.
__device__ __forceinline__ void issue_fence() { asm volatile("" ::: "memory"); }

template <int NT, int MT, int WAVES>
struct PanelGemm {
    static constexpr int kThreads = WAVES * kWave;
    static constexpr int kRows = MT * 16;                       // staged token rows
    static constexpr int kChunks = kPanelCols / 8;              // 16-byte chunks per staged row
    static_assert(kChunks == kWave, "one wave stages one row per instruction");
    static constexpr int kStageLoads = kRows / WAVES;           // rows staged per thread
    static_assert(kRows % WAVES == 0, "rows split evenly over waves");
    static constexpr int kBufElems = kRows * kPanelPitch;
    static constexpr int kLdsElems = 2 * kBufElems;

    // Weight step `step` of this lane's rows into b (clamped to the last block).
    static __device__ __forceinline__ void load_weights(WeightStep (&b)[NT], const uint8_t* __restrict__ w,
                                                        const uint8_t* __restrict__ ws, int K,
                                                        const int (&wrow)[NT], int step) {
        const int g = (threadIdx.x & (kWave - 1)) >> 4;
        const int kblocks = K / 32;
        const int kb0 = min(step * 8 + g, kblocks - 1);
        const int kb1 = min(step * 8 + g + 4, kblocks - 1);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint8_t* rp = w + (size_t)wrow[t] * (K / 2);
            b[t].w[0] = load_nt16(rp + (size_t)kb0 * 16);
            b[t].w[1] = load_nt16(rp + (size_t)kb1 * 16);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint8_t* sp = ws + (size_t)wrow[t] * kblocks;
            b[t].e[0] = sp[kb0];
            b[t].e[1] = sp[kb1];
        }
    }

    // Token rows [0, 16 MTA) of panel `panel` into registers: thread (wave, c)
    // stages 16-byte chunk c of rows wave + WAVES j, whose source rows are
    // src[j].
    template <int MTA>
    static __device__ __forceinline__ void load_panel(u32x4 (&xr)[kStageLoads], const uint16_t* __restrict__ xb,
                                                      size_t xpitch, const int (&src)[kStageLoads], int K,
                                                      int panel) {
        const int c = threadIdx.x & (kWave - 1);
        const int col = min(panel * kPanelCols + 8 * c, K - 8);
#pragma unroll
        for (int j = 0; j < MTA * 16 / WAVES; ++j)
            xr[j] = *reinterpret_cast<const u32x4*>(xb + (size_t)src[j] * xpitch + col);
    }

    template <int MTA>
    static __device__ __forceinline__ void store_panel(const u32x4 (&xr)[kStageLoads], uint16_t* buf) {
        const int c = threadIdx.x & (kWave - 1);
        const int wave = threadIdx.x / kWave;
#pragma unroll
        for (int j = 0; j < MTA * 16 / WAVES; ++j)
            *reinterpret_cast<u32x4*>(buf + (wave + WAVES * j) * kPanelPitch + 8 * c) = xr[j];
    }

    // acc += weight step `step` (held in b) x token panel buffer xs at panel
    // column col0, for token tiles m < MTA. Tiles with tvalid[t] false and
    // blocks past K take zero codes.
    template <int MTA>
    static __device__ __forceinline__ void compute(const WeightStep (&b)[NT], const bool (&tvalid)[NT], int K,
                                                   int step, const uint16_t* xs, int col0, f32x4 (&acc)[NT][MT]) {
        const int lane = threadIdx.x & (kWave - 1);
        const int g = lane >> 4, r = lane & 15;
        const int kblocks = K / 32;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const bool kv = step * 8 + g + 4 * h < kblocks;
            uint32_t wd[NT][4];
            float sc[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const bool ok = kv && tvalid[t];
                const uint4 v = b[t].w[h];
                wd[t][0] = ok ? v.x : 0u;
                wd[t][1] = ok ? v.y : 0u;
                wd[t][2] = ok ? v.z : 0u;
                wd[t][3] = ok ? v.w : 0u;
                sc[t] = e8m0_scale(b[t].e[h]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bf16x8 a[NT];
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const u32x4 u = {fp4x2_to_bf16x2<0>(wd[t][i], sc[t]), fp4x2_to_bf16x2<1>(wd[t][i], sc[t]),
                                     fp4x2_to_bf16x2<2>(wd[t][i], sc[t]), fp4x2_to_bf16x2<3>(wd[t][i], sc[t])};
                    a[t] = __builtin_bit_cast(bf16x8, u);
                }
                const int col = col0 + 32 * (g + 4 * h) + 8 * i;
#pragma unroll
                for (int m = 0; m < MTA; ++m) {
                    const bf16x8 bx = *reinterpret_cast<const bf16x8*>(xs + (16 * m + r) * kPanelPitch + col);
#pragma unroll
                    for (int t = 0; t < NT; ++t)
                        acc[t][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[t], bx, acc[t][m], 0, 0, 0);
                }
            }
        }
    }

    // The whole product over K for one pass of MTA token tiles (16 MTA staged
    // rows, nvalid of them real). lds: kLdsElems bf16; rowidx: LDS list of the
    // pass's source rows, already written and synchronised.
    //
    // Every load below is issued on every path (indices clamped), so the
    // number of loads between any two points is fixed and each wait the
    // compiler places counts exactly the loads issued after the one it needs.
    template <int MTA>
    static __device__ __forceinline__ void run(const uint8_t* __restrict__ w, const uint8_t* __restrict__ ws, int K,
                                               const int (&wrow)[NT], const bool (&tvalid)[NT],
                                               const uint16_t* __restrict__ xb, size_t xpitch, const int* rowidx,
                                               int nvalid, uint16_t* lds, f32x4 (&acc)[NT][MT]) {
        const int npanels = (K + kPanelCols - 1) / kPanelCols;
        const int nsteps = (K + kStepCols - 1) / kStepCols;
        const int wave = threadIdx.x / kWave;
        int src[kStageLoads];
#pragma unroll
        for (int j = 0; j < MTA * 16 / WAVES; ++j) src[j] = rowidx[min(wave + WAVES * j, nvalid - 1)];
        u32x4 xr[kStageLoads];
        WeightStep b0[NT], b1[NT];
        load_panel<MTA>(xr, xb, xpitch, src, K, 0);
        store_panel<MTA>(xr, lds);
        __syncthreads();
        load_weights(b0, w, ws, K, wrow, 0);
        load_weights(b1, w, ws, K, wrow, min(1, nsteps - 1));
        for (int p = 0; p < npanels; ++p) {
            load_panel<MTA>(xr, xb, xpitch, src, K, min(p + 1, npanels - 1));
            issue_fence();
            const uint16_t* xs = lds + (p & 1) * kBufElems;
            compute<MTA>(b0, tvalid, K, 2 * p, xs, 0, acc);
            load_weights(b0, w, ws, K, wrow, min(2 * p + 2, nsteps - 1));
            issue_fence();
            compute<MTA>(b1, tvalid, K, 2 * p + 1, xs, kStepCols, acc);
            load_weights(b1, w, ws, K, wrow, min(2 * p + 3, nsteps - 1));
            issue_fence();
            store_panel<MTA>(xr, lds + ((p + 1) & 1) * kBufElems);
            __syncthreads();
        }
    }

    // run<MTA> for MTA = mt (1 <= mt <= MT), chosen once per pass.
    static __device__ __forceinline__ void run_mt(int mt, const uint8_t* __restrict__ w, const uint8_t* __restrict__ ws,
                                                  int K, const int (&wrow)[NT], const bool (&tvalid)[NT],
                                                  const uint16_t* __restrict__ xb, size_t xpitch, const int* rowidx,
                                                  int nvalid, uint16_t* lds, f32x4 (&acc)[NT][MT]) {
        static_assert(MT == 4, "dispatch written for four token tiles");
        switch (mt) {
            case 1: run<1>(w, ws, K, wrow, tvalid, xb, xpitch, rowidx, nvalid, lds, acc); break;
            case 2: run<2>(w, ws, K, wrow, tvalid, xb, xpitch, rowidx, nvalid, lds, acc); break;
            case 3: run<3>(w, ws, K, wrow, tvalid, xb, xpitch, rowidx, nvalid, lds, acc); break;
            default: run<4>(w, ws, K, wrow, tvalid, xb, xpitch, rowidx, nvalid, lds, acc); break;
        }
    }
};

}  // namespace e2m1
