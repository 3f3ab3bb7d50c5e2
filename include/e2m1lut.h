/*
 * e2m1lut.h -- C ABI of libe2m1lut.so, the MI355X (gfx950) library that
 * decodes packed low-bit weights inside memory-bound matrix-vector and
 * small-batch matrix products.
 *
 * Pages the operations follow (cited by page and section):
 *   [vLLM-51583]   prhub.com.cn digest of vLLM pull request 51583: MXFP4 unpack
 *                  to bf16 by table lookup plus an integer add of the E8M0
 *                  block scale into the bf16 exponent field, both zero codes
 *                  forced to +0.0 ("功能与动机", "实现拆解", "关键源码片段").
 *   [SGLang-34222] prhub.com.cn digest of SGLang pull request 34222: NVFP4
 *                  token embedding dequantised at gather time ("实现拆解",
 *                  "关键源码片段").
 *   [NM-wiki]      sglang-jax wiki page on the N:M structured sparse matmul
 *                  gap ("N:M 稀疏原理", "3.1 Sparsifier", "3.2").
 *   [FairyFuse]    blog.hotdry.top post on FairyFuse: 2-bit ternary GEMV with
 *                  add/sub accumulation and a per-row scale
 *                  ("三元 GEMV 的乘法消除原理"), the widely-linear complex
 *                  layer fused over four ternary matrices
 *                  ("复杂值广泛线性层的融合核调度") and batched ternary GEMM
 *                  for speculative decoding ("总结与启示").
 *
 * Conventions shared by every entry point
 *   - All array pointers are DEVICE pointers (hipMalloc'd or torch CUDA
 *     tensors), owned by the caller, row-major and densely packed. Inputs and
 *     outputs must not overlap.
 *   - `stream` is a hipStream_t passed as void*; NULL means the default
 *     stream. Every call is asynchronous on that stream: nothing allocates,
 *     copies to or from the host, or synchronises. Device-side faults surface
 *     at the caller's next synchronisation.
 *   - Arguments are validated on the host before anything is launched; on a
 *     negative status nothing was launched and no output was written.
 *   - A call whose output is empty (a zero extent) launches nothing and
 *     returns E2M1_OK; pointers may then be NULL.
 *   - Formats:
 *       E2M1 code: 4 bits, bit 3 = sign, bits 0..2 index the magnitudes
 *         {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
 *       Packed code rows: byte j holds column 2j in its low nibble and
 *         column 2j+1 in its high nibble.
 *       E8M0: one uint8 per 32 consecutive columns, value 2^(e-127).
 *       E4M3: OCP float8 e4m3fn (bias 7, no infinities, S.1111.111 = NaN).
 *       bf16 values travel as their uint16 bit patterns.
 */
#ifndef E2M1LUT_H
#define E2M1LUT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define E2M1LUT_ABI_VERSION 2

/* Status codes (0 = success, negative = rejected before launch or launch error). */
#define E2M1_OK 0
#define E2M1_ERR_NULL (-1)      /* a required pointer is NULL */
#define E2M1_ERR_SHAPE (-2)     /* negative extent, or a divisibility / range rule broken */
#define E2M1_ERR_ALIGN (-3)     /* a pointer lacks the alignment the kernel loads need */
#define E2M1_ERR_DTYPE (-4)     /* unknown output dtype code */
#define E2M1_ERR_WORKSPACE (-5) /* workspace missing or smaller than required */
#define E2M1_ERR_LAUNCH (-6)    /* the HIP runtime reported an error at launch (e.g. no gfx950 code for the device) */

/* Output dtype codes for dequant_gemv. */
#define E2M1_DTYPE_F32 0
#define E2M1_DTYPE_BF16 1

/* Largest batch dequant_gemv accepts. */
#define E2M1_GEMV_MAX_BATCH 16

/* Most experts mxfp4_moe_gemm accepts. */
#define E2M1_MOE_MAX_EXPERTS 512

/* ABI version of the loaded library (E2M1LUT_ABI_VERSION it was built with). */
int e2m1_abi_version(void);

/* Static, NUL-terminated description of a status code; never NULL. */
const char* e2m1_strerror(int status);

/*
 * dequant_decode -- unpack an MXFP4 matrix to bf16 bit patterns.
 * Operation: [vLLM-51583] "功能与动机" and "关键源码片段" (vec.h): the code's
 * bf16 pattern from the E2M1 table, plus (e-127)*2^7 added to the 16-bit
 * pattern modulo 2^16; a lane whose table pattern is +0 or -0 is written as
 * +0.0 (0x0000) at every exponent. For 2 <= e <= 252 the result is exactly
 * bf16((+/-)magnitude * 2^(e-127)); outside that range non-zero codes wrap as
 * the integer add dictates (the method's result, not a meaningful value).
 *   packed      uint8  [rows, k/2]   (16-byte aligned)
 *   scale_e8m0  uint8  [rows, k/32]
 *   out_bf16    uint16 [rows, k]     (16-byte aligned), overwritten
 * Requires rows >= 0, k >= 0, k % 32 == 0.
 */
int dequant_decode(const uint8_t* packed, const uint8_t* scale_e8m0, uint16_t* out_bf16,
                   int64_t rows, int64_t k, void* stream);

/*
 * dequant_gemv -- y = x . W^T with W decoded from MXFP4 inside the product.
 * Operation: the decode of dequant_decode followed by a dot product per
 * output, accumulated in fp32 (the unpack feeds the MXFP4 MoE GEMM in
 * [vLLM-51583] "实现拆解" item 2). Defined for E8M0 values 2..252, where the
 * decoded weights are exact; the summation order is unspecified.
 *   packed      uint8  [n, k/2]      (16-byte aligned)
 *   scale_e8m0  uint8  [n, k/32]
 *   x_bf16      uint16 [batch, k]    (bf16 activations, 16-byte aligned)
 *   y           [batch, n], fp32 (y_dtype = E2M1_DTYPE_F32) or bf16 bit
 *               patterns rounded to nearest even (E2M1_DTYPE_BF16);
 *               overwritten, never accumulated into. 4-byte aligned.
 * Requires 1 <= batch <= E2M1_GEMV_MAX_BATCH, n >= 0, k >= 0, k % 32 == 0.
 * k == 0 writes zeros.
 */
int dequant_gemv(const uint8_t* packed, const uint8_t* scale_e8m0, const uint16_t* x_bf16,
                 void* y, int y_dtype, int64_t batch, int64_t n, int64_t k, void* stream);

/* Most matrices one dequant_gemv_grouped call accepts. */
#define E2M1_GEMV_MAX_GROUPS 64

/*
 * dequant_gemv_grouped -- several independent batch-1 dequant_gemv products
 * (matrix g applied to its own activation row) issued together, e.g. the
 * projections of one layer that do not depend on each other. Operation: per
 * matrix exactly that of dequant_gemv at batch 1 ([vLLM-51583] "实现拆解"
 * item 2: the unpack feeding a product); the products share launches (for
 * K <= 16384 one launch holds up to eight matrices), so the fixed cost of a
 * launch is paid once for all their weight bytes.
 *   count                    number of matrices, 0 <= count <= E2M1_GEMV_MAX_GROUPS
 *   packed[g], scale_e8m0[g], x_bf16[g], y[g]
 *                            device pointers laid out as in dequant_gemv with
 *                            batch 1, n = n[g], k = k[g] (same alignments);
 *                            the pointer arrays themselves and n, k are host
 *                            memory, read during the call only
 *   n[g], k[g]               as in dequant_gemv (n >= 0, k >= 0, k % 32 == 0)
 * Every y[g] is overwritten; outputs must not overlap each other or any
 * input. All arguments are validated before anything is launched, so a
 * validation error writes nothing; E2M1_ERR_LAUNCH can follow launches that
 * already ran, and then some outputs are written and others not.
 */
int dequant_gemv_grouped(int count, const uint8_t* const* packed, const uint8_t* const* scale_e8m0,
                         const uint16_t* const* x_bf16, void* const* y, const int64_t* n, const int64_t* k,
                         int y_dtype, void* stream);

/*
 * dequant_gemm -- y = x . W^T for many activation rows (prefill): the MXFP4
 * weight matrix decoded on the way into bf16 matrix-core tiles.
 * Operation: as dequant_gemv ([vLLM-51583] "功能与动机": E2M1 table lookup and
 * E8M0 scale), for any number of rows of x; the page's comment section
 * describes the CPU GEMM decoding weight blocks into bf16 tiles. Accumulation
 * is fp32.
 *   packed      uint8  [n, k/2]   (16-byte aligned)
 *   scale_e8m0  uint8  [n, k/32]
 *   x_bf16      uint16 [m, k]     bf16 patterns (16-byte aligned)
 *   y           [m, n], E2M1_DTYPE_F32 (fp32) or E2M1_DTYPE_BF16 (bf16 RNE), overwritten
 * Requires m, n >= 0, k >= 0, k % 32 == 0, m and n at most 2^31 - 1,
 * k <= E2M1_GEMM_MAX_K (each workgroup addresses its 128 rows of x with 32-bit
 * byte offsets) and fewer than 2^31 tiles of 128 x 128 outputs. k == 0
 * writes zeros. Rows of W or x past n or m are never read.
 */
#define E2M1_GEMM_MAX_K 8388576
int dequant_gemm(const uint8_t* packed, const uint8_t* scale_e8m0, const uint16_t* x_bf16, void* y,
                 int y_dtype, int64_t m, int64_t n, int64_t k, void* stream);

/*
 * nm_spmm -- N:M structured-sparse weights times a few activation rows:
 * y[b][r] = sum over the kept entries of row r of value * x[b][column].
 * Format: [NM-wiki] "N:M 稀疏原理", "3.1 Sparsifier": in every group of M
 * consecutive columns of a row N values are kept; their in-group positions
 * are packed next_log2(M) bits each (1 bit for M = 2), 32 / bits per word,
 * entry i of a row at bit (i mod packing) * bits of word i / packing; rows
 * follow one another. Operation: "3.2" (decompress, then multiply), fp32
 * accumulation.
 *   values   bf16   [rows, (k/M) N]   kept values, group-major (2-byte aligned)
 *   meta     uint32 [rows, ceil((k/M) N / packing)]
 *   x_bf16   bf16   [batch, k]
 *   y        [batch, rows], E2M1_DTYPE_F32 or E2M1_DTYPE_BF16, overwritten
 * Requires 1 <= batch <= 16, 1 <= n_keep <= m_group <= 16, k % m_group == 0,
 * rows, k >= 0 and below 2^31. Positions >= m_group (possible when M is not a
 * power of two) are not valid; the kernel reads them as the group's last
 * column. The fastest kernel takes 2:4, 1:4, 4:8, 1:2 and 8:16 with batch
 * <= 4, (k/M) N % 8 == 0, 16-byte aligned values and x, and k up to about
 * 29000 (one activation row), 15400 (two) or 7700 (three or four), the
 * activations it stages in 64 KB of LDS; everything else takes a slower kernel
 * with the same results up to rounding.
 */
int nm_spmm(const uint16_t* values, const uint32_t* meta, const uint16_t* x_bf16, void* y, int y_dtype,
            int64_t batch, int64_t rows, int64_t k, int n_keep, int m_group, void* stream);

/*
 * mxfp4_quantize -- bf16 rows to MXFP4 codes and E8M0 block scales (the
 * encode side of dequant_decode / dequant_gemv / mxfp4_moe_gemm).
 * Operation: the quantizer the MoE test of [vLLM-51583] "关键源码片段" applies
 * to bf16 weights; the page prints no rounding rule. Rule taken: per 32
 * consecutive columns e = clamp(floor(log2(amax)) - 2 + 127, 0, 254) (0 for an
 * all-zero block); each element becomes the E2M1 code of the value nearest to
 * x / 2^(e-127), ties to the code whose last bit is 0, magnitudes above 6
 * saturating to 6, sign bit from x (so a small negative x gives code 8).
 * Decoding the result returns each element within half an E2M1 step (or 6
 * units, for the elements above 6 units).
 *   x_bf16      uint16 [rows, k]   bf16 patterns (16-byte aligned)
 *   packed      uint8  [rows, k/2] byte j = column 2j (low nibble), 2j+1 (high) (8-byte aligned)
 *   scale_e8m0  uint8  [rows, k/32]
 * Requires rows >= 0, k >= 0, k % 32 == 0; x must be finite.
 */
int mxfp4_quantize(const uint16_t* x_bf16, uint8_t* packed, uint8_t* scale_e8m0, int64_t rows,
                   int64_t k, void* stream);

/*
 * nvfp4_quantize -- bf16 rows to NVFP4 codes and E4M3 block scales for a given
 * fp32 global scale (the encode side of nvfp4_embedding_gather).
 * Operation: [SGLang-34222] "关键源码片段" dequantises value = E2M1 code *
 * fl32(e4m3(block scale) * global); the page prints no encoder. Rule taken:
 * per 16 consecutive columns the block scale byte is the E4M3 value nearest
 * to fl32(amax / fl32(6 * global)), ties to an even mantissa, saturating at
 * 448; eff = fl32(e4m3(bs) * global); each element is the E2M1 code nearest
 * to fl32(x / eff) with the rounding of mxfp4_quantize (eff == 0 gives
 * signed zero codes). Every fp32 step is an IEEE fp32 operation.
 *   x_bf16            uint16 [rows, k]    bf16 patterns (16-byte aligned)
 *   global_scale      fp32   [1] on the device, > 0
 *   packed            uint8  [rows, k/2]  as for mxfp4_quantize (8-byte aligned)
 *   block_scale_e4m3  uint8  [rows, k/16]
 * Requires rows >= 0, k >= 0, k % 16 == 0; x must be finite.
 */
int nvfp4_quantize(const uint16_t* x_bf16, const float* global_scale, uint8_t* packed,
                   uint8_t* block_scale_e4m3, int64_t rows, int64_t k, void* stream);

/*
 * ternary_gemv -- y[i] = row_scale[i] * sum_k t(i,k) * x[k], t in {-1, 0, +1}.
 * Operation: [FairyFuse] "三元 GEMV 的乘法消除原理": 16 weights per uint32,
 * weight j of word w multiplies x[16w + j]; bit 2j+1 set = +1 (add), bit 2j
 * set = -1 (subtract), neither = 0; the per-row scale multiplies once after
 * the row sum. A field with both bits set is not a valid weight; the kernel
 * reads it as 0.
 *   packed     uint32 [n, k/16]  (4-byte aligned)
 *   row_scale  fp32   [n]
 *   x          fp32   [k]        (4-byte aligned)
 *   y          fp32   [n], overwritten
 * Requires n >= 0, k >= 0, k % 16 == 0. k == 0 writes zeros. x must be
 * finite. With k % 64 == 0 and 16-byte aligned packed this is ternary_gemm at
 * batch 1 (exact sums over a fixed-point rendering of x, then a few fp32
 * roundings); other inputs take a slower kernel that adds in fp32.
 */
int ternary_gemv(const uint32_t* packed, const float* row_scale, const float* x, float* y,
                 int64_t n, int64_t k, void* stream);

/*
 * ternary_gemm_workspace_size -- bytes of device workspace ternary_gemm needs
 * for these extents: 0 where it runs without one (batch below 5, k % 64 !=
 * 0, an empty problem), (size_t)-1 for extents ternary_gemm rejects.
 */
size_t ternary_gemm_workspace_size(int64_t batch, int64_t n, int64_t k);

/*
 * ternary_gemm -- small-batch ternary GEMM: y[b][i] = row_scale[i] * sum_k t(i,k) * x[b][k].
 * Operation: [FairyFuse] "三元 GEMV 的乘法消除原理" applied to `batch`
 * activation rows at once, the batched fusion for speculative decoding that
 * "总结与启示" names as the next step; packing and scale as for ternary_gemv.
 *   packed     uint32 [n, k/16]  (4-byte aligned)
 *   row_scale  fp32   [n]
 *   x          fp32   [batch, k] (4-byte aligned)
 *   y          fp32   [batch, n], overwritten (from batch 5: zeroed by the
 *              first launch, then two fp32 atomic adds per element, so it
 *              must be ordinary device memory from hipMalloc)
 *   workspace  device buffer of at least ternary_gemm_workspace_size()
 *              bytes, 256-byte aligned, contents need no initialisation
 *              (may be NULL where that size is 0); the call writes it, so
 *              calls that overlap in time need workspaces of their own
 * Requires 1 <= batch <= E2M1_TERNARY_MAX_BATCH, n >= 0, k >= 0,
 * k % 16 == 0. k == 0 writes zeros. A field with both bits set reads as 0;
 * x must be finite. The fast kernels (k % 64 == 0, 16-byte aligned packed)
 * sum ternary times a fixed-point rendering of x exactly (each element of at
 * least 2^-36 of the largest |x| of its row and 256-column slice exactly, any
 * other to within 2^-60 of that largest) and round in fp32 only a few times
 * per output; from batch 5 on the fixed-point digits are prepared once per
 * call in the workspace by a launch of their own. Other inputs run
 * ternary_gemv once per row of x.
 * Errors: E2M1_ERR_WORKSPACE when a workspace is needed and missing or too
 * small, E2M1_ERR_ALIGN when it is not 256-byte aligned.
 */
#define E2M1_TERNARY_MAX_BATCH 16
int ternary_gemm(const uint32_t* packed, const float* row_scale, const float* x, float* y, void* workspace,
                 size_t workspace_bytes, int64_t batch, int64_t n, int64_t k, void* stream);

/*
 * ternary_wl_gemv -- widely-linear complex ternary layer y = U x + W conj(x).
 * Operation: [FairyFuse] "复杂值广泛线性层的融合核调度": x is complex [k], U
 * and W complex [n, k]; the layer splits into eight real ternary GEMVs, all
 * evaluated in one pass. Each real part is a ternary matrix packed as for
 * ternary_gemv, with its own per-row scale (applied once after the row sum):
 *   U = diag(s_Ure) T_Ure + i diag(s_Uim) T_Uim,  W likewise, so
 *   y_re = s_Ure (T_Ure x_re) - s_Uim (T_Uim x_im) + s_Wre (T_Wre x_re) + s_Wim (T_Wim x_im)
 *   y_im = s_Ure (T_Ure x_im) + s_Uim (T_Uim x_re) - s_Wre (T_Wre x_im) + s_Wim (T_Wim x_re)
 *   packed     HOST array of four DEVICE pointers, in the order U_re, U_im,
 *              W_re, W_im; each uint32 [n, k/16], 4-byte aligned
 *   scale      fp32 [4, n]: the per-row scales, same order
 *   x_re, x_im fp32 [k]
 *   y_re, y_im fp32 [n], overwritten
 * Requires n >= 0, k >= 0, k % 16 == 0. k == 0 writes zeros. A field with
 * both bits set reads as 0. x must be finite: the fast kernel multiplies
 * zero weights by x, so an Inf or NaN in x can turn outputs NaN where the
 * method would skip it. Accumulation is fp32 with x at full fp32 precision.
 * The fast kernel needs k % 64 == 0 and 16-byte aligned matrices; other
 * inputs take a slower kernel with the same results up to rounding.
 */
int ternary_wl_gemv(const uint32_t* const packed[4], const float* scale, const float* x_re,
                    const float* x_im, float* y_re, float* y_im, int64_t n, int64_t k, void* stream);

/*
 * nvfp4_embedding_gather -- gather token rows of an NVFP4 table and
 * dequantise them to bf16.
 * Operation: [SGLang-34222] "实现拆解" item 2 and "关键源码片段"
 * (embedding()): for output row i and column c with r = ids[i]: the code is
 * the low nibble of table[r, c/2] for even c and the high nibble for odd c;
 * v = (+/-)magnitude in fp32 (code 8 is -0.0, sign kept); eff =
 * fp32(e4m3(block_scale[r, c/16]) * global_scale); out = bf16_rne(fp32(v *
 * eff)). NaN results are written as 0x7FC0.
 *   table             uint8  [vocab, hidden/2]   (8-byte aligned; 16-byte
 *                     alignment and hidden % 32 == 0 select the widest loads)
 *   block_scale_e4m3  uint8  [vocab, hidden/16]
 *   global_scale      fp32   [1] on the device (read by the kernel, so the
 *                     call needs no host synchronisation)
 *   ids               int64  [num_tokens]
 *   out_bf16          uint16 [num_tokens, hidden], overwritten (16-byte aligned)
 *   err_flag          int32  [1] on the device, or NULL. An id outside
 *                     [0, vocab) gives an all-zero output row and, when
 *                     err_flag is given, stores 1 there (never cleared by
 *                     the library).
 * Requires vocab >= 0, hidden >= 0, hidden % 16 == 0 (the page's
 * create_weights divisibility guard), num_tokens >= 0. With vocab == 0 the
 * table and block_scale may be NULL and are never read: every id is out of
 * range, so every row is written as zeros and err_flag is set.
 */
int nvfp4_embedding_gather(const uint8_t* table, const uint8_t* block_scale_e4m3,
                           const float* global_scale, const int64_t* ids, uint16_t* out_bf16,
                           int64_t vocab, int64_t hidden, int64_t num_tokens, int32_t* err_flag,
                           void* stream);

/*
 * mxfp4_moe_workspace_size -- bytes of device workspace mxfp4_moe_gemm needs
 * for these extents (0 for an empty problem; (size_t)-1 for invalid extents).
 */
size_t mxfp4_moe_workspace_size(int64_t tokens, int64_t hidden, int64_t inter, int64_t experts,
                                int64_t topk);

/*
 * mxfp4_moe_gemm -- MXFP4 mixture-of-experts layer with routing as input.
 * Operation: the fused expert op exercised by [vLLM-51583] "关键源码片段"
 * (the MoE test): per token t and slot j, e = topk_ids[t, j]:
 *   h = W13[e] . x_t (2*inter outputs; rows [0, inter) gate, [inter, 2*inter) up),
 *   a = silu(gate) * up, y = W2[e] . a,
 *   out[t] = bf16_rne(sum_j topk_weights[t, j] * y).
 * Products run on bf16 MFMA with fp32 accumulation; `a` is rounded to bf16
 * before the second product. The combine over slots runs in slot order
 * (deterministic).
 *   x              uint16 [tokens, hidden]  bf16
 *   w13            uint8  [experts, 2*inter, hidden/2]   (16-byte aligned)
 *   w13_scale      uint8  [experts, 2*inter, hidden/32]
 *   w2             uint8  [experts, hidden, inter/2]     (16-byte aligned)
 *   w2_scale       uint8  [experts, hidden, inter/32]
 *   topk_ids       int32  [tokens, topk], each in [0, experts)
 *   topk_weights   fp32   [tokens, topk]
 *   out            uint16 [tokens, hidden]  bf16, overwritten
 *   workspace      device buffer of at least mxfp4_moe_workspace_size()
 *                  bytes, 256-byte aligned; contents need no initialisation
 * Requires hidden % 32 == 0, inter % 32 == 0, 1 <= experts <=
 * E2M1_MOE_MAX_EXPERTS, topk >= 1, tokens >= 0, tokens * topk <= INT_MAX,
 * inter * hidden < 2^31 (each expert's W13 below 2 GiB).
 * Ids outside [0, experts) are not checked on the host (they live on the
 * device); the kernels skip such slots (they contribute nothing).
 */
int mxfp4_moe_gemm(const uint16_t* x, const uint8_t* w13, const uint8_t* w13_scale,
                   const uint8_t* w2, const uint8_t* w2_scale, const int32_t* topk_ids,
                   const float* topk_weights, uint16_t* out, void* workspace,
                   size_t workspace_bytes, int64_t tokens, int64_t hidden, int64_t inter,
                   int64_t experts, int64_t topk, void* stream);

/*
 * mxfp4_moe_gemm_noalloc -- mxfp4_moe_gemm for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. Same operation, arguments (minus the workspace),
 * layouts, kernels and results as mxfp4_moe_gemm; the workspace is instead a
 * fixed array inside the library, E2M1_MOE_NOALLOC_WORKSPACE_BYTES per GPU,
 * which every GPU the library is loaded on holds until the process ends. The
 * call allocates nothing (no hipMalloc, no library allocation).
 * Returns E2M1_ERR_WORKSPACE, before touching the GPU, when
 * mxfp4_moe_workspace_size() of the extents exceeds that maximum (32 MiB:
 * up to 485 tokens at top-4 with hidden = inter = 2880). Every call on one GPU
 * shares that GPU's array, which keeps the last call's contents (the layer
 * needs none of it to start at zero): calls that overlap on one GPU (on other
 * streams or from other host threads) race and must be serialised by the
 * caller.
 */
#define E2M1_MOE_NOALLOC_WORKSPACE_BYTES ((size_t)32 << 20)
int mxfp4_moe_gemm_noalloc(const uint16_t* x, const uint8_t* w13, const uint8_t* w13_scale,
                           const uint8_t* w2, const uint8_t* w2_scale, const int32_t* topk_ids,
                           const float* topk_weights, uint16_t* out, int64_t tokens,
                           int64_t hidden, int64_t inter, int64_t experts, int64_t topk,
                           void* stream);

#ifdef __cplusplus
}
#endif

#endif /* E2M1LUT_H */
