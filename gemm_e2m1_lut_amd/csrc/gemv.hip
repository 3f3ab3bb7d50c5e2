// gemv.hip -- MXFP4 dequant-GEMV / small-batch GEMM (dequant_gemv).
//
// y[b, n] = sum_k W[n, k] x[b, k], W decoded from E2M1 codes with an E8M0
// scale per 32 columns (the unpack of the vLLM pull request 51583 digest,
// sections "功能与动机" and "实现拆解": the unpack feeds the MXFP4 MoE GEMM),
// accumulated in fp32.
//
// gfx950 design.
//   * Decode: v_cvt_scalef32_pk_bf16_fp4 turns one byte (two codes) into two
//     bf16 already multiplied by the block scale 2^(e-127); for 2 <= e <= 252
//     these are exactly the bf16 patterns of the lookup + exponent-add unpack
//     (zero codes give +/-0, which add nothing to a sum). v_dot2_f32_bf16
//     multiplies the pair by the matching pair of x and accumulates in fp32:
//     per byte of weights one conversion and one dot2.
//   * Batch 1 (the bandwidth-bound case): every load instruction reads one
//     row x 1 KB contiguous (lane l the 16-byte chunk l of a 64-chunk slice),
//     each lane's slice of x sits in registers, and every weight load of a
//     wave is issued before its first use. Up to K = 4096 a single wave owns
//     four whole rows (two chunks per lane at K = 4096), so nothing passes
//     through LDS; up to K = 16384 a workgroup of S = K / 2048 waves owns 16
//     rows, wave w the slice w, and the S partial row sums meet in LDS. The row
//     sums of a wave come out of one transposed reduction over its 64 lanes
//     (v_permlane32_swap, v_permlane16_swap and DPP). Every weight byte is read
//     once. Longer rows (K > 16384) are split over the waves of a workgroup,
//     one chunk per lane, with three rows in flight; short rows (K <= 1024)
//     use groups of 8 to 32 lanes per row.
//   * Batch 2..4 with 1024 < K <= 16384: a workgroup of S = K / 1024 waves
//     owns 16 rows, each load instruction reads two rows x 512 bytes, and the
//     B activation rows sit side by side in registers: B dot2 per decoded
//     pair.
//   * Batch 2..16 otherwise (batch 5..16, or K <= 1024): the same weight
//     bytes feed bf16 MFMA (v_mfma_f32_16x16x32_bf16) with the batch as the
//     N dimension: a workgroup takes a tile of 16 rows, its S waves split K
//     into slices of 1024 columns; each wave loads its code lines coalesced
//     (eight rows x 128 bytes per instruction) and turns them into A operands
//     through a per-wave LDS transpose, and stages each half step's x columns
//     in LDS for the B operands (rows past the batch and columns past the
//     row end read as zero). Every weight byte is still read once; the S
//     partial 16 x 16 tiles meet in LDS and are summed in a fixed order.
//   * K beyond the tiled kernels (K > 16384 at batch 2..16, K > 32768 at
//     batch 1): one wave per row, lanes across K, x read per chunk.
#include "device.hpp"
#include "kernels.hpp"

namespace e2m1 {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;

// Dot product of one 32-column block (16 code bytes in w, scale s) with the 16
// x words (bf16 pairs) of the same columns. Two accumulators halve the
// dependency chain.
__device__ __forceinline__ float block_dot(const uint4 w, float s, const uint32_t* xw, float acc) {
    float a0 = 0.f, a1 = 0.f;
    a0 = dot2_bf16(fp4x2_to_bf16x2<0>(w.x, s), xw[0], a0);
    a1 = dot2_bf16(fp4x2_to_bf16x2<1>(w.x, s), xw[1], a1);
    a0 = dot2_bf16(fp4x2_to_bf16x2<2>(w.x, s), xw[2], a0);
    a1 = dot2_bf16(fp4x2_to_bf16x2<3>(w.x, s), xw[3], a1);
    a0 = dot2_bf16(fp4x2_to_bf16x2<0>(w.y, s), xw[4], a0);
    a1 = dot2_bf16(fp4x2_to_bf16x2<1>(w.y, s), xw[5], a1);
    a0 = dot2_bf16(fp4x2_to_bf16x2<2>(w.y, s), xw[6], a0);
    a1 = dot2_bf16(fp4x2_to_bf16x2<3>(w.y, s), xw[7], a1);
    a0 = dot2_bf16(fp4x2_to_bf16x2<0>(w.z, s), xw[8], a0);
    a1 = dot2_bf16(fp4x2_to_bf16x2<1>(w.z, s), xw[9], a1);
    a0 = dot2_bf16(fp4x2_to_bf16x2<2>(w.z, s), xw[10], a0);
    a1 = dot2_bf16(fp4x2_to_bf16x2<3>(w.z, s), xw[11], a1);
    a0 = dot2_bf16(fp4x2_to_bf16x2<0>(w.w, s), xw[12], a0);
    a1 = dot2_bf16(fp4x2_to_bf16x2<1>(w.w, s), xw[13], a1);
    a0 = dot2_bf16(fp4x2_to_bf16x2<2>(w.w, s), xw[14], a0);
    a1 = dot2_bf16(fp4x2_to_bf16x2<3>(w.w, s), xw[15], a1);
    return acc + (a0 + a1);
}

template <bool kBf16Out>
__device__ __forceinline__ void store_out(void* y, int64_t idx, float v) {
    if constexpr (kBf16Out)
        reinterpret_cast<uint16_t*>(y)[idx] = (uint16_t)f32_to_bf16_rne(v);
    else
        reinterpret_cast<float*>(y)[idx] = v;
}

// ------------------------------------------------------------- batch 1 ----

// Row total of groups of G lanes (G in {8, 16, 32, 64}) with DPP only: the
// total ends up in the last lane of each group (lane G-1 mod G).
template <int G>
__device__ __forceinline__ float group_total(float v) {
    v += dpp_f32<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp_f32<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp_f32<0x141>(v);   // row_half_mirror: every lane holds its 8-lane sum
    if constexpr (G >= 16) v += dpp_f32<0x140>(v);   // row_mirror: 16-lane sum
    if constexpr (G >= 32)   // row_bcast:15 into rows 1 and 3
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
    if constexpr (G >= 64)   // row_bcast:31 into rows 2 and 3
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));
    return v;
}

// Totals of N per-lane values over aligned groups of 2^(Top+1) lanes (Top = 4:
// each half wave; Top = 5: the whole wave), reduced as a transposed butterfly.
// Stage s (s = Top .. 0) pairs every lane with one whose lane-index bit s
// differs (bit 5 through v_permlane32_swap, bit 4 through v_permlane16_swap,
// bits 3..0 through the DPP row mirror, half-row mirror and quad
// permutations); while a lane holds an even number m of values it halves
// them, the lane with bit s clear keeping the pair sums of values [0, m/2)
// and the other those of [m/2, m); with an odd m it adds its partner's values
// to all of its own. On return v[0 .. lane_totals_count<Top, N>()) of lane L
// hold the totals of value indices lane_totals_base<Top, N>(L) + j, and lanes
// that differ only in the low lane_totals_dup_bits<Top, N>() bits of the lane
// index hold the same ones. Against one DPP reduction per value this costs
// about 2.5 instead of 5 or 6 operations per value for N >= 8, and the
// independent pairs of a stage fill the DPP wait states.
template <int Top, int N>
constexpr int lane_totals_count() {
    int m = N;
    for (int st = Top; st >= 0; --st)
        if (m % 2 == 0) m /= 2;
    return m;
}

template <int Top, int N>
constexpr int lane_totals_dup_bits() {
    int m = N, bits = 0;
    for (int st = Top; st >= 0; --st) {
        if (m % 2 == 0) m /= 2;
        else ++bits;
    }
    return bits;
}

template <int Top, int N>
__device__ __forceinline__ int lane_totals_base(int lane) {
    int m = N, base = 0;
#pragma unroll
    for (int st = Top; st >= 0; --st)
        if (m % 2 == 0) {
            m /= 2;
            base += ((lane >> st) & 1) * m;
        }
    return base;
}

template <int St>
__device__ __forceinline__ float lane_partner(float v) {   // lane-index bit St flipped, St < 4
    if constexpr (St == 3) return dpp_f32<0x140>(v);   // row_mirror: lane i <-> 15 - i
    if constexpr (St == 2) return dpp_f32<0x141>(v);   // row_half_mirror: i <-> 7 - i
    if constexpr (St == 1) return dpp_f32<0x4E>(v);    // quad_perm [2,3,0,1]
    return dpp_f32<0xB1>(v);                           // quad_perm [1,0,3,2]
}

// a + b exchanged across lane-index bit St (5 or 4): lanes with the bit clear
// get a(L) + a(L ^ 2^St), lanes with it set b(L ^ 2^St) + b(L).
template <int St>
__device__ __forceinline__ float swap_sum(float a, float b) {
    if constexpr (St == 5) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    } else {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
}

template <int St, int M>
__device__ __forceinline__ void lane_totals_stage(float* v, int lane) {
    if constexpr (M % 2 == 0) {
        constexpr int H = M / 2;
        const bool upper = (lane >> St) & 1;
#pragma unroll
        for (int j = 0; j < H; ++j) {
            if constexpr (St >= 4) {   // the swap leaves v[j] pairs on bit-clear lanes, v[j + H] pairs on the others
                v[j] = swap_sum<St>(v[j], v[j + H]);
            } else {
                const float keep = upper ? v[j + H] : v[j];
                const float send = upper ? v[j] : v[j + H];
                v[j] = keep + lane_partner<St>(send);
            }
        }
        if constexpr (St > 0) lane_totals_stage<St - 1, H>(v, lane);
    } else {
#pragma unroll
        for (int j = 0; j < M; ++j) {
            if constexpr (St >= 4) v[j] = swap_sum<St>(v[j], v[j]);
            else v[j] += lane_partner<St>(v[j]);
        }
        if constexpr (St > 0) lane_totals_stage<St - 1, M>(v, lane);
    }
}

template <int Top, int N>
__device__ __forceinline__ void lane_totals(float (&v)[N], int lane) {
    lane_totals_stage<Top, N>(v, lane);
}

// Batch 1. A group of G lanes covers one row; lane gl owns the 32-column chunks
// gl, gl + G, ... (CPL of them) for every row it visits, so its slice of x is
// loaded once into registers. A group takes R consecutive rows per pass. All
// loads are unconditional (indices clamped into range, out-of-range lanes and
// rows masked at use): guarded loads with a zero in the other branch would
// make each load wait for the previous one. x is requested first, then every
// weight chunk and scale of the pass, so computing row 0 waits only for x and
// row 0 while the later rows are still in flight.
template <int G, int CPL, int R, bool kBf16Out>
__global__ __launch_bounds__(kThreads) void gemv_b1_kernel(const uint8_t* __restrict__ packed,
                                                           const uint8_t* __restrict__ scales,
                                                           const uint16_t* __restrict__ x,
                                                           void* __restrict__ y, int n, int kc) {
    constexpr int kGroupsPerWave = kWave / G;
    const int lane = threadIdx.x & (kWave - 1);
    const int gl = lane & (G - 1);
    const int grp = lane / G;
    const int wave = blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    const int units = gridDim.x * kWavesPerBlock * kGroupsPerWave;   // row groups in the grid
    const int unit = wave * kGroupsPerWave + grp;
    const uint4* xv = reinterpret_cast<const uint4*>(x);
    const uint4* pv = reinterpret_cast<const uint4*>(packed);

    uint32_t xr[CPL][16];
#pragma unroll
    for (int ci = 0; ci < CPL; ++ci) {
        const int c = min(gl + G * ci, kc - 1);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 v = xv[c * 4 + q];
            xr[ci][4 * q + 0] = v.x;
            xr[ci][4 * q + 1] = v.y;
            xr[ci][4 * q + 2] = v.z;
            xr[ci][4 * q + 3] = v.w;
        }
    }
    // wave-uniform pass count: passes while the wave's first group has rows
    for (int pass = 0; (pass * units + wave * kGroupsPerWave) * R < n; ++pass) {
        const int row0 = (pass * units + unit) * R;
        uint4 w[R][CPL];
        uint32_t e[R][CPL];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int ci = 0; ci < CPL; ++ci) {
                const int64_t blk = (int64_t)min(row0 + r, n - 1) * kc + min(gl + G * ci, kc - 1);
                w[r][ci] = load_nt16(pv + blk);
                e[r][ci] = scales[blk];
            }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float acc = 0.f;
#pragma unroll
            for (int ci = 0; ci < CPL; ++ci) {
                const uint4 wv = (gl + G * ci < kc) ? w[r][ci] : make_uint4(0u, 0u, 0u, 0u);
                acc = block_dot(wv, e8m0_scale(e[r][ci]), xr[ci], acc);
            }
            acc = group_total<G>(acc);
            if (gl == G - 1 && row0 + r < n) store_out<kBf16Out>(y, row0 + r, acc);
        }
    }
}

// Keeps loads where they are written (issued early) instead of letting the
// compiler sink them next to their uses; emits no instruction. The weight
// pointers of the kernels that rely on it are not __restrict__: loads through
// a restrict pointer to read-only memory may be moved across the fence.
__device__ __forceinline__ void issue_here() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

template <int CPL>
struct RowBuf {
    uint4 w[CPL];
    uint8_t e[CPL];   // kept as bytes: widened at use, so no instruction touches a pending load
};

// x words of 32-column chunk min(c, kc - 1) (16 bf16 pairs). Lanes whose
// chunk lies past the row end drop their partial sums at use instead (a
// select here would make the first weight loads wait for x).
__device__ __forceinline__ void load_x_chunk(uint32_t (&xr)[16], const uint16_t* __restrict__ x, int c, int kc) {
    const uint4* xv = reinterpret_cast<const uint4*>(x) + 4 * min(c, kc - 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint4 v = xv[q];
        xr[4 * q + 0] = v.x;
        xr[4 * q + 1] = v.y;
        xr[4 * q + 2] = v.z;
        xr[4 * q + 3] = v.w;
    }
}

// Batch 1, 32 < K/32 <= 512: a workgroup of S waves owns R consecutive rows;
// wave w covers the chunks 64 (CPL w + i) + l (i < CPL) of every row, lane l
// taking those with index l, so each load instruction reads one row x 1 KB
// contiguous (the fastest read pattern of the platform: one row per
// instruction instead of two half rows, a quarter fewer x bytes per weight
// byte at K = 4096). x for the lane's chunks is loaded once, before the
// weights (loads complete in order, so the first block waits only for x and
// its own line). Chunks past the row end are loaded clamped and their partial
// sums dropped (E2M1 codes times a clamped E8M0 scale are always finite). The
// R row sums of a wave come out of one transposed reduction over the 64
// lanes; with S = 1 (K <= 64 CPL chunks, one wave per four whole rows, no LDS
// and no barrier) the lanes that hold them store directly, otherwise the S
// wave partials meet in LDS and are summed in a fixed order.
// The tile of rows row0 .. row0 + R - 1 for wave wv of S (part: S x R floats
// of LDS shared by the S waves; unused when S == 1).
template <int S, int CPL, int R, bool kBf16Out>
__device__ __forceinline__ void b1_rows_tile(const uint8_t* packed, const uint8_t* scales,
                                             const uint16_t* __restrict__ x, void* __restrict__ y, int n,
                                             int kc, int row0, int wv, int lane, float (*part)[R]) {
    const uint4* pv = reinterpret_cast<const uint4*>(packed);
    int c[CPL];
    bool cvalid[CPL];
    uint32_t xr[CPL][16];
#pragma unroll
    for (int ci = 0; ci < CPL; ++ci) {
        const int c_raw = (wv * CPL + ci) * kWave + lane;
        cvalid[ci] = c_raw < kc;
        c[ci] = min(c_raw, kc - 1);
        load_x_chunk(xr[ci], x, c_raw, kc);
    }
    issue_here();
    uint4 w[CPL][R];
    uint8_t e[CPL][R];   // kept as bytes: widened at use
#pragma unroll
    for (int ci = 0; ci < CPL; ++ci)
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t blk = (int64_t)min(row0 + r, n - 1) * kc + c[ci];
            w[ci][r] = load_nt16(pv + blk);
            e[ci][r] = scales[blk];
        }
    issue_here();
    float tot[R];
#pragma unroll
    for (int r = 0; r < R; ++r) tot[r] = 0.f;
#pragma unroll
    for (int ci = 0; ci < CPL; ++ci)
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float p = block_dot(w[ci][r], e8m0_scale(e[ci][r]), xr[ci], 0.f);
            tot[r] += cvalid[ci] ? p : 0.f;
        }
    lane_totals<5>(tot, lane);   // lane L: totals of rows base + j
    constexpr int kDup = lane_totals_dup_bits<5, R>();
    const int base = lane_totals_base<5, R>(lane);
    if constexpr (S == 1) {
        if ((lane & ((1 << kDup) - 1)) == 0) {
#pragma unroll
            for (int j = 0; j < lane_totals_count<5, R>(); ++j)
                if (row0 + base + j < n) store_out<kBf16Out>(y, row0 + base + j, tot[j]);
        }
    } else {
        if ((lane & ((1 << kDup) - 1)) == 0) {
#pragma unroll
            for (int j = 0; j < lane_totals_count<5, R>(); ++j) part[wv][base + j] = tot[j];
        }
        __syncthreads();
        if (threadIdx.x < R) {
            float sum = 0.f;
#pragma unroll
            for (int j = 0; j < S; ++j) sum += part[j][threadIdx.x];
            const int row = row0 + threadIdx.x;
            if (row < n) store_out<kBf16Out>(y, row, sum);
        }
    }
}

template <int S, int CPL, int R, bool kBf16Out>
__global__ __launch_bounds__(kWave * S) void gemv_b1_rows_kernel(const uint8_t* packed, const uint8_t* scales,
                                                                 const uint16_t* __restrict__ x,
                                                                 void* __restrict__ y, int n, int kc) {
    __shared__ float part[S][R];
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    b1_rows_tile<S, CPL, R, kBf16Out>(packed, scales, x, y, n, kc, blockIdx.x * R, wv, lane, part);
}

// Several independent batch-1 products in one launch (e.g. the projections of
// one layer that read the same or different activations): the fixed cost of a
// launch (dispatch, ramp-up, drain and the final write-back, about 1.5-2 us
// here) is paid once for all their weight bytes instead of once per matrix.
// Each matrix keeps the tiling it gets alone: K <= 2048 / 4096 as S
// independent one-wave tiles of four whole rows per workgroup (kind 0 / 1),
// 4096 < K <= 16384 as one 16-row tile of S waves (kind 2, every such matrix
// of a launch needing the same S). Workgroups map to matrices through
// ascending first-block indices (scalar, uniform per workgroup).
constexpr int kGroupMax = 8;
constexpr int kGroupRows = 16;   // rows of a multi-wave tile
struct B1Group {
    const uint8_t* packed;
    const uint8_t* scales;
    const uint16_t* x;
    void* y;
    int n, kc, kind, block0;
};
struct B1GroupSet {
    B1Group g[kGroupMax];
    int count;
};

template <int S, bool kBf16Out>
__global__ __launch_bounds__(kWave * S) void gemv_b1_group_kernel(const B1GroupSet set) {
    __shared__ float part[S][kGroupRows];
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int blk = blockIdx.x;
    B1Group g = set.g[0];   // constant indices only: the selection stays in scalar registers
#pragma unroll
    for (int i = 1; i < kGroupMax; ++i)
        if (i < set.count && blk >= set.g[i].block0) g = set.g[i];
    const int local = blk - g.block0;
    if (g.kind == 2) {
        b1_rows_tile<S, 1, kGroupRows, kBf16Out>(g.packed, g.scales, g.x, g.y, g.n, g.kc, local * kGroupRows, wv,
                                                 lane, part);
        return;
    }
    const int row0 = (local * S + wv) * 4;   // one-wave tiles: wave-uniform exit past the last row
    if (row0 >= g.n) return;
    if (g.kind == 0)
        b1_rows_tile<1, 1, 4, kBf16Out>(g.packed, g.scales, g.x, g.y, g.n, g.kc, row0, 0, lane, nullptr);
    else
        b1_rows_tile<1, 2, 4, kBf16Out>(g.packed, g.scales, g.x, g.y, g.n, g.kc, row0, 0, lane, nullptr);
}

// Batch 2..4, 32 < K/32 <= 32 S: one workgroup of S waves per tile of 16
// rows, lane l taking chunk 32 w + l % 32 of rows 2 q + l / 32 (two rows x
// 512 contiguous bytes per load instruction), with the B activation rows'
// words of the lane's chunk in registers: each
// decoded code pair meets them in B v_dot2_f32_bf16, so the decode is shared
// by the batch and nothing but the row totals passes through LDS. The work
// per weight byte grows with B (one conversion, B dot2 and B shares of the
// row reductions), which is why from five rows on the matrix-core kernel
// below takes over.
template <int S, int B, bool kBf16Out>
__global__ __launch_bounds__(kWave * S) void gemv_bn_tile_kernel(const uint8_t* packed, const uint8_t* scales,
                                                                 const uint16_t* __restrict__ x,
                                                                 void* __restrict__ y, int n, int kc) {
    __shared__ float part[S][B][16];
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int half = lane >> 5, cl = lane & 31;
    const int c_raw = wv * 32 + cl;
    const bool cvalid = c_raw < kc;
    const int c = min(c_raw, kc - 1);
    const uint4* pv = reinterpret_cast<const uint4*>(packed);
    uint32_t xr[B][16];
#pragma unroll
    for (int b = 0; b < B; ++b) load_x_chunk(xr[b], x + (size_t)b * kc * 32, c, kc);
    issue_here();
    const int tile = blockIdx.x;
    uint4 w[8];
    uint8_t e[8];   // kept as bytes: widened at use
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int row = min(tile * 16 + 2 * q + half, n - 1);
        const int64_t blk = (int64_t)row * kc + c;
        w[q] = load_nt16(pv + blk);
        e[q] = scales[blk];
    }
    issue_here();
    float tot[8 * B];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const float s = e8m0_scale(e[q]);
        const uint32_t ws[4] = {w[q].x, w[q].y, w[q].z, w[q].w};
        uint32_t wd[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            wd[4 * i + 0] = fp4x2_to_bf16x2<0>(ws[i], s);
            wd[4 * i + 1] = fp4x2_to_bf16x2<1>(ws[i], s);
            wd[4 * i + 2] = fp4x2_to_bf16x2<2>(ws[i], s);
            wd[4 * i + 3] = fp4x2_to_bf16x2<3>(ws[i], s);
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
            float a = 0.f;
#pragma unroll
            for (int j = 0; j < 16; ++j) a = dot2_bf16(wd[j], xr[b][j], a);
            tot[8 * b + q] = cvalid ? a : 0.f;
        }
    }
    lane_totals<4>(tot, lane);   // lane L: totals of value indices base + j = 8 b + q
    if ((lane & ((1 << lane_totals_dup_bits<4, 8 * B>()) - 1)) == 0) {
        const int base = lane_totals_base<4, 8 * B>(lane);
#pragma unroll
        for (int j = 0; j < lane_totals_count<4, 8 * B>(); ++j) {
            const int idx = base + j;
            part[wv][idx / 8][2 * (idx % 8) + half] = tot[j];
        }
    }
    __syncthreads();
    if (threadIdx.x < 16 * B) {
        const int b = threadIdx.x / 16, r = threadIdx.x % 16;
        float sum = 0.f;
#pragma unroll
        for (int j = 0; j < S; ++j) sum += part[j][b][r];
        const int row = tile * 16 + r;
        if (row < n) store_out<kBf16Out>(y, (int64_t)b * n + row, sum);
    }
}

// Batch 1, K/32 > 512: rows split over the S waves of a workgroup, lane l of
// wave w owning chunk 64 w + l. Rows blockIdx.x + i * gridDim.x, three in
// flight per wave (buffer r % 4 for row r, loop started three rows early as
// above); the S partial totals of each row meet in LDS, 64 rows at a time,
// and are summed in a fixed order.
template <int S, bool kBf16Out>
__global__ __launch_bounds__(kWave * S) void gemv_b1_split_kernel(const uint8_t* packed,
                                                                  const uint8_t* scales,
                                                                  const uint16_t* __restrict__ x,
                                                                  void* __restrict__ y, int n, int kc) {
    constexpr int kDepth = 3;
    constexpr int kBufs = kDepth + 1;
    __shared__ float part[S][kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int c_raw = wv * kWave + lane;
    const int c = min(c_raw, kc - 1);
    const int nb = gridDim.x;
    const int row0 = blockIdx.x;
    const uint4* pv = reinterpret_cast<const uint4*>(packed);

    uint32_t xr[16];
    load_x_chunk(xr, x, c_raw, kc);
    issue_here();
    const int iters = (n - 1 - row0) / nb + 1;   // grid <= n: at least one row
    const int last = row0 + (iters - 1) * nb;
    RowBuf<1> buf[kBufs];
    float res = 0.f;
    for (int it = -kDepth; it < iters; it += kBufs) {
#pragma unroll
        for (int b = 0; b < kBufs; ++b) {
            const int i = it + b;   // row being summed; row i + 3 is issued into buffer b
            {
                const int64_t blk = (int64_t)min(row0 + (i + kDepth) * nb, last) * kc + c;
                buf[b].w[0] = load_nt16(pv + blk);
                buf[b].e[0] = scales[blk];
            }
            issue_here();
            if (i >= 0 && i < iters) {   // workgroup-uniform
                const RowBuf<1>& cur = buf[(b + 1) % kBufs];
                const float p = block_dot(cur.w[0], e8m0_scale(cur.e[0]), xr, 0.f);
                const float acc = group_total<kWave>(c_raw < kc ? p : 0.f);
                const float t = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc), kWave - 1));
                const int slot = i & (kWave - 1);
                if (lane == slot) res = t;
                if (slot == kWave - 1 || i == iters - 1) {
                    part[wv][lane] = res;
                    __syncthreads();
                    if ((int)threadIdx.x <= slot) {
                        float s = 0.f;
#pragma unroll
                        for (int j = 0; j < S; ++j) s += part[j][threadIdx.x];
                        store_out<kBf16Out>(y, (int64_t)row0 + (int64_t)(i - slot + threadIdx.x) * nb, s);
                    }
                    __syncthreads();
                }
            }
            issue_here();
        }
    }
}

// ------------------------------------------------------- batch 2..16 ----

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kTileSteps = 4;                        // 256-column steps per wave slice
constexpr int kSliceBlocks = 8 * kTileSteps;         // 32 scale blocks = 1024 columns per wave
constexpr int kMaxSliceWaves = 16;

constexpr int kXPitch = 128 + 8;                     // bf16 per staged x row (16-byte pad spreads the banks)
constexpr int kWPitch = 9;                           // uint4 per transposed code row (8 blocks + pad)

// Workgroup = S waves on one tile of 16 RT rows (tiles blockIdx.x, +
// gridDim.x, ...); wave w owns scale blocks [32 w, 32 w + 32) of all of them,
// and each staged x operand serves the RT 16-row MFMA tiles. Lane l = 16 g + r: row r
// of the tile for the A operand and batch column r for the B operand; in half
// step hs = 2 s + h it loads block b = 32 w + 8 s + g + 4 h (the two halves of
// a 128-byte line of the row are half steps h = 0, 1). MFMA (hs, i) takes
// codes [8 i, 8 i + 8) of block b as A k-slots 8 g .. 8 g + 7 and the same
// columns of x as B k-slots, so both operands share one column -> k-slot map
// and the sum over k is complete. D element (row 4 g + j, batch r) is
// component j of acc in lane l.
// x reaches the B operands through the wave's own LDS area: the half step's
// 128 columns of all batch rows are loaded with coalesced 16-byte loads (16
// lanes per 256-byte row, NJ = ceil(batch / 4) loads per lane), written to
// LDS and read back per MFMA; loading them per lane straight from memory
// would make each B operand a separate 16-byte request into a different row
// of x. The x loads of half step 0 go out first, then every weight load of the
// slice, then the x loads of half step hs + 1 right after half step hs is
// staged; one wave writes and reads its own area, and LDS accesses of a wave
// complete in order, so no barrier is needed.
template <bool kBf16Out, int NJ, int RT, int kMaxW>
__global__ __launch_bounds__(kWave * kMaxW) void gemv_mfma_kernel(
    const uint8_t* packed, const uint8_t* scales, const uint16_t* x, void* __restrict__ y,
    int batch, int n, int kc) {
    __shared__ f32x4 part[RT][kMaxW][kWave];
    extern __shared__ __attribute__((aligned(16))) uint16_t gemv_xs[];
    constexpr int kXRows = 4 * NJ;
    constexpr int kHalfSteps = 2 * kTileSteps;
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int nwaves = blockDim.x / kWave;
    const int r = lane & 15, g = lane >> 4;
    const int K = kc * 32;
    const int ntiles = (n + 16 * RT - 1) / (16 * RT);
    const bool bvalid = r < batch;
    uint16_t* xs = gemv_xs + wv * (kXRows * kXPitch + 8 * kWPitch * 16 * RT);
    uint4* wbuf = reinterpret_cast<uint4*>(xs + kXRows * kXPitch);   // RT x 16 rows x kWPitch uint4
    // staging: chunk j of a lane is row 4 j + (lane >> 4), columns 8 (lane & 15) .. + 7 of the half step
    uint16_t* xdst = xs + (lane >> 4) * kXPitch + 8 * (lane & 15);
    const uint16_t* xread = xs + min(r, batch - 1) * kXPitch + 32 * g;
    // x through a buffer resource of exactly batch * K elements: the hardware
    // range check returns zeros for the rows past the batch and the columns past
    // the last row (columns past K on earlier rows read the next row, in blocks
    // whose B operand is masked). One 32-bit lane offset serves every load;
    // per-load address pairs would be hoisted out of the tile loop and pinned.
    const __amdgpu_buffer_rsrc_t xres =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), 0, batch * K * 2, kBufferWord3);
    const int xlane = 2 * ((lane >> 4) * K + 8 * (lane & 15));
    auto load_x = [&](uint4 (&xg)[NJ], int hs) {
        const int col = wv * kSliceBlocks * 32 + hs * 128;
        int xl = xlane;
        asm volatile("" : "+v"(xl));   // offsets are formed here, not kept for every half step
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(xres, xl + 2 * (4 * j * K + col), 0, 0);
            xg[j] = make_uint4(v.x, v.y, v.z, v.w);
        }
    };

    for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {   // workgroup-uniform
        const uint8_t* srow[RT];
#pragma unroll
        for (int t = 0; t < RT; ++t)
            srow[t] = scales + (size_t)min(tile * 16 * RT + 16 * t + r, n - 1) * kc;
        uint4 xg[NJ];
        load_x(xg, 0);
        issue_here();
        // scale bytes straight in MFMA layout, then the code lines: load (st, q) of lane l is row
        // 8 q + l / 8 of the tile, block 8 st + l % 8 (eight rows x 128 contiguous bytes per
        // instruction). Loads complete in order: with the scales first, half step 2 st waits only
        // for the lines of steps <= st, so the first MFMAs overlap the later lines' arrival
        // (scales last: 14.0 -> 12.9 us at batch 8, 17.3 -> 15.8 at batch 16, 14336 x 4096).
        uint4 wl[kTileSteps][RT][2];
        uint32_t e[RT][kHalfSteps];
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int hs = 0; hs < kHalfSteps; ++hs)
                e[t][hs] = srow[t][min(wv * kSliceBlocks + 8 * (hs >> 1) + g + 4 * (hs & 1), kc - 1)];
        issue_here();
        const uint8_t* lrow[RT][2];
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int q = 0; q < 2; ++q)
                lrow[t][q] = packed + (size_t)min(tile * 16 * RT + 16 * t + 8 * q + (lane >> 3), n - 1) * (K / 2);
#pragma unroll
        for (int st = 0; st < kTileSteps; ++st) {
            const int b = min(wv * kSliceBlocks + 8 * st + (lane & 7), kc - 1);
#pragma unroll
            for (int t = 0; t < RT; ++t)
#pragma unroll
                for (int q = 0; q < 2; ++q) wl[st][t][q] = load_nt16(lrow[t][q] + (size_t)b * 16);
        }
        issue_here();
        f32x4 acc[RT];
#pragma unroll
        for (int t = 0; t < RT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        uint4 wm[RT][2];   // this step's blocks g and g + 4 of row r of each tile (MFMA layout)
#pragma unroll
        for (int hs = 0; hs < kHalfSteps; ++hs) {
            if ((hs & 1) == 0) {   // a new step: its code lines through the wave's LDS transpose
#pragma unroll
                for (int t = 0; t < RT; ++t)
#pragma unroll
                    for (int q = 0; q < 2; ++q)
                        wbuf[(16 * t + 8 * q + (lane >> 3)) * kWPitch + (lane & 7)] = wl[hs >> 1][t][q];
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j) *reinterpret_cast<uint4*>(xdst + 4 * j * kXPitch) = xg[j];
            issue_here();   // the registers are free before the next half step's loads reuse them
            if (hs + 1 < kHalfSteps) load_x(xg, hs + 1);
            issue_here();
            __builtin_amdgcn_wave_barrier();
            if ((hs & 1) == 0) {
#pragma unroll
                for (int t = 0; t < RT; ++t) {
                    wm[t][0] = wbuf[(16 * t + r) * kWPitch + g];
                    wm[t][1] = wbuf[(16 * t + r) * kWPitch + g + 4];
                }
            }
            const bool valid = bvalid && (wv * kSliceBlocks + 8 * (hs >> 1) + g + 4 * (hs & 1) < kc);
            float sc[RT];
            uint32_t ws[RT][4];
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                sc[t] = e8m0_scale(e[t][hs]);
                const uint4 wh = wm[t][hs & 1];
                ws[t][0] = wh.x;
                ws[t][1] = wh.y;
                ws[t][2] = wh.z;
                ws[t][3] = wh.w;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u32x4 xv = *reinterpret_cast<const u32x4*>(xread + 8 * i);
                const u32x4 bz = {valid ? xv.x : 0u, valid ? xv.y : 0u, valid ? xv.z : 0u, valid ? xv.w : 0u};
#pragma unroll
                for (int t = 0; t < RT; ++t) {
                    const u32x4 a = {fp4x2_to_bf16x2<0>(ws[t][i], sc[t]), fp4x2_to_bf16x2<1>(ws[t][i], sc[t]),
                                     fp4x2_to_bf16x2<2>(ws[t][i], sc[t]), fp4x2_to_bf16x2<3>(ws[t][i], sc[t])};
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                                      __builtin_bit_cast(bf16x8, bz), acc[t], 0, 0, 0);
                }
            }
            __builtin_amdgcn_wave_barrier();   // this half step's reads come before the next writes
        }
#pragma unroll
        for (int t = 0; t < RT; ++t) part[t][wv][lane] = acc[t];
        __syncthreads();
        // thread i sums element (row 16 t + 4 g + j, batch c) over the slices: i = 256 t + 64 j + 16 g + c
        for (int i = threadIdx.x; i < 4 * kWave * RT; i += blockDim.x) {
            const int t = i / (4 * kWave), j = (i / kWave) & 3, l = i & (kWave - 1);
            const int c = l & 15, orow = tile * 16 * RT + 16 * t + 4 * (l >> 4) + j;
            float sum = 0.f;
            for (int q = 0; q < nwaves; ++q) sum += part[t][q][l][j];
            if (c < batch && orow < n) store_out<kBf16Out>(y, (int64_t)c * n + orow, sum);
        }
        __syncthreads();
    }
}

// --------------------------------------------------------- any batch ----

template <int B, bool kBf16Out>
__global__ __launch_bounds__(kThreads) void gemv_generic_kernel(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ scales,
    const uint16_t* __restrict__ x, void* __restrict__ y, int n, int kc) {
    const int lane = threadIdx.x & (kWave - 1);
    const int nwaves = gridDim.x * kWavesPerBlock;
    const uint4* xv = reinterpret_cast<const uint4*>(x);
    for (int row = blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; row < n; row += nwaves) {
        float acc[B];
#pragma unroll
        for (int b = 0; b < B; ++b) acc[b] = 0.f;
        for (int c = lane; c < kc; c += kWave) {
            const int64_t blk = (int64_t)row * kc + c;
            const uint4 w = load_nt16(reinterpret_cast<const uint4*>(packed) + blk);
            const float s = e8m0_scale(scales[blk]);
            uint32_t wd[16];
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                wd[4 * q + 0] = fp4x2_to_bf16x2<0>(ws[q], s);
                wd[4 * q + 1] = fp4x2_to_bf16x2<1>(ws[q], s);
                wd[4 * q + 2] = fp4x2_to_bf16x2<2>(ws[q], s);
                wd[4 * q + 3] = fp4x2_to_bf16x2<3>(ws[q], s);
            }
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const uint4* xp = xv + ((int64_t)b * kc + c) * 4;
                float a = acc[b];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint4 xq = xp[q];
                    a = dot2_bf16(wd[4 * q + 0], xq.x, a);
                    a = dot2_bf16(wd[4 * q + 1], xq.y, a);
                    a = dot2_bf16(wd[4 * q + 2], xq.z, a);
                    a = dot2_bf16(wd[4 * q + 3], xq.w, a);
                }
                acc[b] = a;
            }
        }
#pragma unroll
        for (int b = 0; b < B; ++b) acc[b] = group_sum<kWave>(acc[b]);
        if (lane == 0) {
#pragma unroll
            for (int b = 0; b < B; ++b) store_out<kBf16Out>(y, (int64_t)b * n + row, acc[b]);
        }
    }
}

// ------------------------------------------------------------- launch ----

template <typename Kernel>
int resident_blocks(Kernel kernel, size_t lds_bytes, int threads = kThreads) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds_bytes) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    return per_cu * device_cu_count();
}

template <int G, int CPL, int R, bool kBf16Out>
hipError_t run_b1_r(const uint8_t* packed, const uint8_t* scales, const uint16_t* x, void* y, int n,
                    int kc, int cap, hipStream_t stream) {
    const int rows_per_block = kWavesPerBlock * (kWave / G) * R;
    const int want = (n + rows_per_block - 1) / rows_per_block;
    const int grid = want < cap ? want : cap;
    gemv_b1_kernel<G, CPL, R, kBf16Out><<<grid, kThreads, 0, stream>>>(packed, scales, x, y, n, kc);
    return hipGetLastError();
}

// Rows per group and pass: the fewest (1, 2 or 4) that let every row group of
// one resident wave generation finish the matrix in a single pass.
template <int G, int CPL, bool kBf16Out>
hipError_t run_b1(const uint8_t* packed, const uint8_t* scales, const uint16_t* x, void* y, int n,
                  int kc, hipStream_t stream) {
    static int cap1 = 0, cap2 = 0, cap4 = 0;   // resident blocks per R, same on every gfx950
    if (cap1 == 0) {
        cap1 = resident_blocks(gemv_b1_kernel<G, CPL, 1, kBf16Out>, 0);
        cap2 = resident_blocks(gemv_b1_kernel<G, CPL, 2, kBf16Out>, 0);
        cap4 = resident_blocks(gemv_b1_kernel<G, CPL, 4, kBf16Out>, 0);
    }
    const int groups_per_block = kWavesPerBlock * (kWave / G);
    if ((int64_t)cap1 * groups_per_block >= n)
        return run_b1_r<G, CPL, 1, kBf16Out>(packed, scales, x, y, n, kc, cap1, stream);
    if ((int64_t)cap2 * groups_per_block * 2 >= n || CPL > 4)
        return run_b1_r<G, CPL, 2, kBf16Out>(packed, scales, x, y, n, kc, cap2, stream);
    return run_b1_r<G, CPL, 4, kBf16Out>(packed, scales, x, y, n, kc, cap4, stream);
}

template <int S, int CPL, int R, bool kBf16Out>
hipError_t run_b1_rows(const uint8_t* packed, const uint8_t* scales, const uint16_t* x, void* y, int n, int kc,
                       hipStream_t stream) {
    const int blocks = (n + R - 1) / R;   // one workgroup per R rows
    gemv_b1_rows_kernel<S, CPL, R, kBf16Out><<<blocks, kWave * S, 0, stream>>>(packed, scales, x, y, n, kc);
    return hipGetLastError();
}

template <int S, int B, bool kBf16Out>
hipError_t run_bn_tile(const uint8_t* packed, const uint8_t* scales, const uint16_t* x, void* y, int n, int kc,
                       hipStream_t stream) {
    const int tiles = (n + 15) / 16;   // one workgroup per tile of 16 rows
    gemv_bn_tile_kernel<S, B, kBf16Out><<<tiles, kWave * S, 0, stream>>>(packed, scales, x, y, n, kc);
    return hipGetLastError();
}

template <int B, bool kBf16Out>
hipError_t dispatch_bn(const uint8_t* packed, const uint8_t* scales, const uint16_t* x, void* y, int n, int kc,
                       hipStream_t stream) {
    switch ((kc + 31) / 32) {
#define E2M1_TILE_CASE(S) \
    case S: return run_bn_tile<S, B, kBf16Out>(packed, scales, x, y, n, kc, stream);
        E2M1_TILE_CASE(2) E2M1_TILE_CASE(3) E2M1_TILE_CASE(4) E2M1_TILE_CASE(5) E2M1_TILE_CASE(6)
        E2M1_TILE_CASE(7) E2M1_TILE_CASE(8) E2M1_TILE_CASE(9) E2M1_TILE_CASE(10) E2M1_TILE_CASE(11)
        E2M1_TILE_CASE(12) E2M1_TILE_CASE(13) E2M1_TILE_CASE(14) E2M1_TILE_CASE(15)
        default: return run_bn_tile<16, B, kBf16Out>(packed, scales, x, y, n, kc, stream);
#undef E2M1_TILE_CASE
    }
}

template <int S, bool kBf16Out>
hipError_t run_b1_split(const uint8_t* packed, const uint8_t* scales, const uint16_t* x, void* y, int n, int kc,
                        hipStream_t stream) {
    const int grid = min(n, device_cu_count());   // one workgroup of S waves per compute unit
    gemv_b1_split_kernel<S, kBf16Out><<<grid, kWave * S, 0, stream>>>(packed, scales, x, y, n, kc);
    return hipGetLastError();
}

template <bool kBf16Out>
hipError_t dispatch_b1(const uint8_t* packed, const uint8_t* scales, const uint16_t* x, void* y,
                       int n, int kc, hipStream_t stream) {
    if (kc <= 8) return run_b1<8, 1, kBf16Out>(packed, scales, x, y, n, kc, stream);
    if (kc <= 16) return run_b1<16, 1, kBf16Out>(packed, scales, x, y, n, kc, stream);
    if (kc <= 32) return run_b1<32, 1, kBf16Out>(packed, scales, x, y, n, kc, stream);
    // one wave per four whole rows (14336 x 4096: 6.6 us per launch against 6.7
    // for 16-row tiles of two half-row waves)
    if (kc <= 64) return run_b1_rows<1, 1, 4, kBf16Out>(packed, scales, x, y, n, kc, stream);
    if (kc <= 128) return run_b1_rows<1, 2, 4, kBf16Out>(packed, scales, x, y, n, kc, stream);
    switch ((kc + kWave - 1) / kWave) {   // 16-row tiles, one 64-chunk slice per wave
        case 3: return run_b1_rows<3, 1, 16, kBf16Out>(packed, scales, x, y, n, kc, stream);
        case 4: return run_b1_rows<4, 1, 16, kBf16Out>(packed, scales, x, y, n, kc, stream);
        case 5: return run_b1_rows<5, 1, 16, kBf16Out>(packed, scales, x, y, n, kc, stream);
        case 6: return run_b1_rows<6, 1, 16, kBf16Out>(packed, scales, x, y, n, kc, stream);
        case 7: return run_b1_rows<7, 1, 16, kBf16Out>(packed, scales, x, y, n, kc, stream);
        case 8: return run_b1_rows<8, 1, 16, kBf16Out>(packed, scales, x, y, n, kc, stream);
        // K > 16384: row slabs streamed through 9..16 waves
        case 9: return run_b1_split<9, kBf16Out>(packed, scales, x, y, n, kc, stream);
        case 10: return run_b1_split<10, kBf16Out>(packed, scales, x, y, n, kc, stream);
        case 11: return run_b1_split<11, kBf16Out>(packed, scales, x, y, n, kc, stream);
        case 12: return run_b1_split<12, kBf16Out>(packed, scales, x, y, n, kc, stream);
        case 13: return run_b1_split<13, kBf16Out>(packed, scales, x, y, n, kc, stream);
        case 14: return run_b1_split<14, kBf16Out>(packed, scales, x, y, n, kc, stream);
        case 15: return run_b1_split<15, kBf16Out>(packed, scales, x, y, n, kc, stream);
        default: return run_b1_split<16, kBf16Out>(packed, scales, x, y, n, kc, stream);
    }
}

template <int B, bool kBf16Out>
hipError_t run_generic(const uint8_t* packed, const uint8_t* scales, const uint16_t* x, void* y,
                       int n, int kc, hipStream_t stream) {
    auto kernel = gemv_generic_kernel<B, kBf16Out>;
    const int want = (n + kWavesPerBlock - 1) / kWavesPerBlock;
    static int cap = 0;
    if (cap == 0) cap = resident_blocks(kernel, 0);
    const int grid = want < cap ? want : cap;
    kernel<<<grid, kThreads, 0, stream>>>(packed, scales, x, y, n, kc);
    return hipGetLastError();
}

template <bool kBf16Out>
hipError_t dispatch_generic(int batch, const uint8_t* packed, const uint8_t* scales,
                            const uint16_t* x, void* y, int n, int kc, hipStream_t stream) {
#define E2M1_GEMV_CASE(B) \
    case B: return run_generic<B, kBf16Out>(packed, scales, x, y, n, kc, stream);
    switch (batch) {
        E2M1_GEMV_CASE(1) E2M1_GEMV_CASE(2) E2M1_GEMV_CASE(3) E2M1_GEMV_CASE(4)
        E2M1_GEMV_CASE(5) E2M1_GEMV_CASE(6) E2M1_GEMV_CASE(7) E2M1_GEMV_CASE(8)
        E2M1_GEMV_CASE(9) E2M1_GEMV_CASE(10) E2M1_GEMV_CASE(11) E2M1_GEMV_CASE(12)
        E2M1_GEMV_CASE(13) E2M1_GEMV_CASE(14) E2M1_GEMV_CASE(15) E2M1_GEMV_CASE(16)
        default: return hipErrorInvalidValue;
    }
#undef E2M1_GEMV_CASE
}

template <bool kBf16Out, int NJ, int RT, int kMaxW>
hipError_t run_mfma_cfg(int batch, const uint8_t* packed, const uint8_t* scales, const uint16_t* x, void* y,
                        int n, int kc, hipStream_t stream) {
    const int waves = (kc + kSliceBlocks - 1) / kSliceBlocks;
    const int ntiles = (n + 16 * RT - 1) / (16 * RT);
    const size_t lds = (size_t)waves * (4 * NJ * kXPitch * sizeof(uint16_t) + 16 * RT * kWPitch * sizeof(uint4));
    static int cache[kMaxSliceWaves + 1] = {};   // resident workgroups per compute unit, per wave count
    int& per_cu = cache[waves];
    if (per_cu == 0) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(gemv_mfma_kernel<kBf16Out, NJ, RT, kMaxW>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, gemv_mfma_kernel<kBf16Out, NJ, RT, kMaxW>,
                                                         kWave * waves, lds) != hipSuccess ||
            per_cu < 1)
            per_cu = 1;
    }
    const int grid = min(ntiles, per_cu * device_cu_count());
    gemv_mfma_kernel<kBf16Out, NJ, RT, kMaxW><<<grid, kWave * waves, lds, stream>>>(packed, scales, x, y, batch, n, kc);
    return hipGetLastError();
}

// Up to eight waves (K <= 8192): two 16-row tiles per wave, so each staged x
// operand serves two MFMAs and every x byte is read once per 32 rows; more
// waves (128 VGPRs each at 16 waves) keep one tile per wave.
template <bool kBf16Out, int NJ>
hipError_t run_mfma_nj(int batch, const uint8_t* packed, const uint8_t* scales, const uint16_t* x, void* y,
                       int n, int kc, hipStream_t stream) {
    const int waves = (kc + kSliceBlocks - 1) / kSliceBlocks;
    if (waves <= 8) return run_mfma_cfg<kBf16Out, NJ, 2, 8>(batch, packed, scales, x, y, n, kc, stream);
    return run_mfma_cfg<kBf16Out, NJ, 1, kMaxSliceWaves>(batch, packed, scales, x, y, n, kc, stream);
}

template <bool kBf16Out>
hipError_t run_mfma(int batch, const uint8_t* packed, const uint8_t* scales, const uint16_t* x, void* y, int n,
                    int kc, hipStream_t stream) {
    switch ((batch + 3) / 4) {   // x loads per lane and half step: four batch rows per 64-lane load
        case 1: return run_mfma_nj<kBf16Out, 1>(batch, packed, scales, x, y, n, kc, stream);
        case 2: return run_mfma_nj<kBf16Out, 2>(batch, packed, scales, x, y, n, kc, stream);
        case 3: return run_mfma_nj<kBf16Out, 3>(batch, packed, scales, x, y, n, kc, stream);
        default: return run_mfma_nj<kBf16Out, 4>(batch, packed, scales, x, y, n, kc, stream);
    }
}

template <int S, bool kBf16Out>
hipError_t run_b1_group(const B1GroupSet& set, int blocks, hipStream_t stream) {
    gemv_b1_group_kernel<S, kBf16Out><<<blocks, kWave * S, 0, stream>>>(set);
    return hipGetLastError();
}

// One launch of up to kGroupMax matrices whose multi-wave tiles (kind 2) all
// have S waves; S also sets how many one-wave tiles a workgroup of kind 0 / 1
// holds.
template <bool kBf16Out>
hipError_t launch_b1_set(const GemvMatrix* const* mats, int count, int S, hipStream_t stream) {
    B1GroupSet set{};
    set.count = count;
    int64_t blocks = 0;
    int slot = 0;
    // multi-wave tiles take the first block indices: the dispatcher starts
    // them first, and the shorter one-wave workgroups fill the slots around
    // them (issued after them, the one-wave blocks would fill the machine
    // and the long tiles would run alone at the end)
    for (int pass = 0; pass < 2; ++pass)
        for (int i = 0; i < count; ++i) {
            const GemvMatrix& m = *mats[i];
            const int kc = (int)(m.k / 32), n = (int)m.n;
            const int kind = kc <= 64 ? 0 : kc <= 128 ? 1 : 2;
            if ((kind == 2) != (pass == 0)) continue;
            set.g[slot++] = B1Group{m.packed, m.scales, m.x, m.y, n, kc, kind, (int)blocks};
            blocks += kind == 2 ? (n + kGroupRows - 1) / kGroupRows : (n + 4 * S - 1) / (4 * S);
        }
    if (blocks * kWave * S > (int64_t)UINT32_MAX) return hipErrorInvalidValue;   // grid past the launch limit
    switch (S) {
        case 3: return run_b1_group<3, kBf16Out>(set, blocks, stream);
        case 5: return run_b1_group<5, kBf16Out>(set, blocks, stream);
        case 6: return run_b1_group<6, kBf16Out>(set, blocks, stream);
        case 7: return run_b1_group<7, kBf16Out>(set, blocks, stream);
        case 8: return run_b1_group<8, kBf16Out>(set, blocks, stream);
        default: return run_b1_group<4, kBf16Out>(set, blocks, stream);
    }
}

}  // namespace

// Largest K of the batch-1 kernels: 16 waves of 64 lanes, one 32-column chunk
// per lane (whole rows per wave stop at 4 chunks per lane, K = 8192).
constexpr int64_t kB1MaxK = 16 * 64 * 32;

hipError_t launch_gemv(const uint8_t* packed, const uint8_t* scales, const uint16_t* x, void* y,
                       bool out_bf16, int batch, int64_t n, int64_t k, hipStream_t stream) {
    const int kc = (int)(k / 32);
    const int nn = (int)n;
    if (batch == 1 && k <= kB1MaxK)
        return out_bf16 ? dispatch_b1<true>(packed, scales, x, y, nn, kc, stream)
                        : dispatch_b1<false>(packed, scales, x, y, nn, kc, stream);
    if (batch >= 2 && batch <= 4 && kc > 32 && kc <= kMaxSliceWaves * kSliceBlocks) {
        if (batch == 4)
            return out_bf16 ? dispatch_bn<4, true>(packed, scales, x, y, nn, kc, stream)
                            : dispatch_bn<4, false>(packed, scales, x, y, nn, kc, stream);
        if (batch == 2)
            return out_bf16 ? dispatch_bn<2, true>(packed, scales, x, y, nn, kc, stream)
                            : dispatch_bn<2, false>(packed, scales, x, y, nn, kc, stream);
        return out_bf16 ? dispatch_bn<3, true>(packed, scales, x, y, nn, kc, stream)
                        : dispatch_bn<3, false>(packed, scales, x, y, nn, kc, stream);
    }
    if (batch > 1 && kc <= kMaxSliceWaves * kSliceBlocks)
        return out_bf16 ? run_mfma<true>(batch, packed, scales, x, y, nn, kc, stream)
                        : run_mfma<false>(batch, packed, scales, x, y, nn, kc, stream);
    return out_bf16 ? dispatch_generic<true>(batch, packed, scales, x, y, nn, kc, stream)
                    : dispatch_generic<false>(batch, packed, scales, x, y, nn, kc, stream);
}

// Matrices with K > 16384 run alone (their kernels stream row slabs); the
// others share launches, one per distinct multi-wave tile width S.
hipError_t launch_gemv_group(const GemvMatrix* mats, int count, bool out_bf16, hipStream_t stream) {
    const GemvMatrix* pend[kGroupMax];
    for (int i = 0; i < count; ++i)
        if (mats[i].k > 16 * 1024) {
            const hipError_t err = launch_gemv(mats[i].packed, mats[i].scales, mats[i].x, mats[i].y, out_bf16, 1,
                                               mats[i].n, mats[i].k, stream);
            if (err != hipSuccess) return err;
        }
    bool done[kGemvGroupMax] = {};
    for (int first = 0; first < count; ++first) {
        if (done[first] || mats[first].k > 16 * 1024) continue;
        // the launch's S: that of the first pending multi-wave matrix, else 4
        int S = 4;
        for (int i = first; i < count; ++i) {
            const int kc = (int)(mats[i].k / 32);
            if (!done[i] && kc > 128 && kc <= 512) { S = (kc + 63) / 64; break; }
        }
        int np = 0;
        for (int i = first; i < count && np < kGroupMax; ++i) {
            const int kc = (int)(mats[i].k / 32);
            if (done[i] || kc > 512 || (kc > 128 && (kc + 63) / 64 != S)) continue;
            pend[np++] = &mats[i];
            done[i] = true;
        }
        const hipError_t err = out_bf16 ? launch_b1_set<true>(pend, np, S, stream)
                                        : launch_b1_set<false>(pend, np, S, stream);
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace e2m1
