/*
 * oracle.c -- plain, slow CPU oracle for the low-bit dequantisation hot path.
 *
 * TEST INFRASTRUCTURE ONLY. This is the reference the HIP library is checked
 * against. Only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark may load it; the product path never does. It shares no code,
 * header, table or constant generator with the HIP library: every table below
 * is a literal written from the pages, and every helper is private to this
 * file.
 *
 * Pages followed (cited by page and section; no line numbers):
 *   [vLLM-51583]    prhub.com.cn digest of vLLM pull request 51583 (CPU MXFP4
 *                   unpack: the zero-code special case folded into fewer
 *                   instructions, bit-exact). Sections "功能与动机"
 *                   (motivation), "实现拆解" (implementation breakdown) and
 *                   "关键源码片段" (key source excerpts: vec.h and the MoE test).
 *   [SGLang-34222]  prhub.com.cn digest of SGLang pull request 34222 (NVFP4
 *                   token embedding, dequantised at gather time). Sections
 *                   "实现拆解" and "关键源码片段" (modelopt_quant.py excerpt and
 *                   the test's element-loop reference).
 *   [NM-wiki]       sglang-jax wiki page on the gap "N:M structured sparse
 *                   matmul" (tpu-inference's Sparsifier and sparse matmul).
 *                   Sections "N:M 稀疏原理", "3.1 Sparsifier" and "3.2".
 *   [FairyFuse]     blog.hotdry.top post on FairyFuse (fused ternary kernels,
 *                   multiplication-free CPU inference). Sections
 *                   "三元 GEMV 的乘法消除原理" (ternary GEMV without multiplies),
 *                   "复杂值广泛线性层的融合核调度" (the widely-linear complex
 *                   layer) and "总结与启示" (batched GEMM for speculative
 *                   decoding as the next step).
 *
 * Arithmetic is fp64 throughout except the NVFP4 gather, whose page fixes
 * fp32 (both scale factors are cast to float and multiplied in float before
 * the final bf16 cast). Loops are scalar; OpenMP splits rows or tokens only,
 * never a sum, so every result is independent of the thread count.
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared -ffp-contract=off (no fast-math).
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#if FLT_EVAL_METHOD != 0
#error "the NVFP4 reference needs float expressions evaluated in float"
#endif

#define OR_OK 0
#define OR_EINVAL (-1)   /* bad shape, or an input the method leaves undefined */
#define OR_ENOMEM (-2)

/* E2M1 magnitudes, indexed by the low three bits of a 4-bit code; bit 3 is
 * the sign. Printed as a lookup table in [SGLang-34222] "关键源码片段" (both
 * the implementation and its test print the same eight values). */
static const double E2M1_MAGNITUDE[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

int or_abi_version(void) { return 1; }

int or_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the loops that follow (n >= 1); results do not depend on it. */
void or_set_threads(int n) {
#ifdef _OPENMP
    omp_set_num_threads(n > 0 ? n : 1);
#else
    (void)n;
#endif
}

double or_e2m1_magnitude(int index) { return E2M1_MAGNITUDE[index & 7]; }

/* ---------------------------------------------------------------- bf16 --- */

/* bf16 bit pattern of a double, rounded once, to nearest with ties to even.
 * Definition: bf16 has 7 stored fraction bits and the fp32 exponent range;
 * below 2^-126 the spacing stays 2^-133 (subnormals). Values that round to
 * 2^128 or beyond become infinity; NaN becomes the canonical quiet NaN. */
uint16_t or_bf16_from_double(double v) {
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0x0000;
    double a = fabs(v);
    if (a == 0.0) return sign;
    if (isinf(a)) return (uint16_t)(sign | 0x7F80);
    int e2;
    (void)frexp(a, &e2);            /* a = f * 2^e2 with f in [0.5, 1) */
    int E = e2 - 1;                 /* a lies in [2^E, 2^(E+1)) */
    if (E < -126) E = -126;         /* subnormal: fixed spacing */
    int q = E - 7;                  /* spacing of representable values is 2^q */
    double r = nearbyint(ldexp(a, -q));   /* default mode: ties to even */
    double vr = ldexp(r, q);
    if (vr >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80);
    float f = (float)vr;            /* exact: <= 8 significant bits, in range */
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    return (uint16_t)(sign | (uint16_t)(bits >> 16));
}

double or_double_from_bf16(uint16_t h) {
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

void or_bf16_from_double_array(const double* in, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = or_bf16_from_double(in[i]);
}

/* ---------------------------------------------------------------- E4M3 --- */

/* OCP FP8 E4M3 ("fn" variant): 1 sign, 4 exponent bits with bias 7, 3
 * fraction bits, subnormals when the exponent field is 0, no infinities, and
 * S.1111.111 is NaN. [SGLang-34222] "实现拆解" names the block scale as e4m3
 * but prints only its cast to float; this decoding is the format's
 * published definition. */
double or_e4m3_to_double(uint8_t b) {
    int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
    if (e == 15 && m == 7) return NAN;
    double v = (e == 0) ? ldexp((double)m, -9)          /* m/8 * 2^(1-7) */
                        : ldexp((double)(8 + m), e - 10); /* (1+m/8) * 2^(e-7) */
    return s ? -v : v;
}

/* --------------------------------------------------------------- MXFP4 --- */

/* 4-bit code of column c of a packed row: byte c/2 holds column 2j in its
 * low nibble and column 2j+1 in its high nibble ([SGLang-34222]
 * "关键源码片段": even channels take the low four bits). */
static int code_at(const uint8_t* row, int64_t c) {
    uint8_t byte = row[c / 2];
    return (c % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
}

/* bf16 pattern of the E2M1 value of a code, sign included (-0 for code 8). */
static uint16_t e2m1_bf16(int code) {
    double m = E2M1_MAGNITUDE[code & 7];
    return or_bf16_from_double((code & 8) ? -m : m);
}

/* The MXFP4 -> bf16 unpack of [vLLM-51583]: look the code up in the bf16
 * table, then apply the E8M0 block scale as an integer add of (e-127) to the
 * bf16 exponent field, i.e. add (e-127)*2^7 to the 16-bit pattern modulo
 * 2^16 ("功能与动机"; "关键源码片段", vec.h). The two zero codes have no
 * exponent to shift, so a lane whose pattern is zero apart from the sign is
 * written as +0.0 (same sections; the excerpt states both zero codes map to
 * +0.0). For 2 <= e <= 252 the result is exactly the bf16 of
 * (+/-)magnitude * 2^(e-127); outside that range a non-zero code's exponent
 * field leaves 1..254 and the integer add wraps, which the page's own test
 * avoids. */
uint16_t or_mxfp4_decode_one(int code, int e8m0) {
    uint16_t base = e2m1_bf16(code & 15);
    if ((base & 0x7FFF) == 0) return 0x0000;
    uint16_t addend = (uint16_t)((e8m0 - 127) * 128);
    return (uint16_t)(base + addend);
}

/* Decode a packed MXFP4 matrix: packed [rows, k/2], one E8M0 byte per 32
 * consecutive columns in scales [rows, k/32], out [rows, k] bf16 patterns. */
int or_mxfp4_decode(const uint8_t* packed, const uint8_t* scales, uint16_t* out,
                    int64_t rows, int64_t k) {
    if (rows < 0 || k < 0 || k % 32 != 0) return OR_EINVAL;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const uint8_t* prow = packed + r * (k / 2);
        const uint8_t* srow = scales + r * (k / 32);
        for (int64_t c = 0; c < k; ++c)
            out[r * k + c] = or_mxfp4_decode_one(code_at(prow, c), srow[c / 32]);
    }
    return OR_OK;
}

/* Real value of one MXFP4 weight: (+/-)magnitude * 2^(e-127), the quantity
 * the unpack above represents exactly for 2 <= e <= 252. */
static double mxfp4_value(int code, int e8m0) {
    double m = E2M1_MAGNITUDE[code & 7];
    return ldexp((code & 8) ? -m : m, e8m0 - 127);
}

/* y[b, r] = sum_c W[r, c] * x[b, c] in fp64, for packed W [n, k] and bf16 x
 * [batch, k]. Every product is exact in fp64; the sum runs in column order.
 * The caller rounds y to the output type. */
int or_mxfp4_gemv(const uint8_t* packed, const uint8_t* scales, const uint16_t* x,
                  double* y, int64_t batch, int64_t n, int64_t k) {
    if (batch < 0 || n < 0 || k < 0 || k % 32 != 0) return OR_EINVAL;
    int fail = 0;
#pragma omp parallel reduction(| : fail)
    {
        double* w = (double*)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
        if (!w) {
            fail = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t r = 0; r < n; ++r) {
                const uint8_t* prow = packed + r * (k / 2);
                const uint8_t* srow = scales + r * (k / 32);
                for (int64_t c = 0; c < k; ++c) w[c] = mxfp4_value(code_at(prow, c), srow[c / 32]);
                for (int64_t b = 0; b < batch; ++b) {
                    double acc = 0.0;
                    for (int64_t c = 0; c < k; ++c) acc += w[c] * or_double_from_bf16(x[b * k + c]);
                    y[b * n + r] = acc;
                }
            }
            free(w);
        }
    }
    return fail ? OR_ENOMEM : OR_OK;
}

/* ------------------------------------------------------------- ternary --- */

/* Ternary GEMV of [FairyFuse] "三元 GEMV 的乘法消除原理": sixteen weights per
 * 32-bit word, weight j of word i multiplies x[16i + j]; bit 2j+1 set means
 * +1 (add x), bit 2j set means -1 (subtract x), neither means 0. The only
 * multiply is the per-row scale, applied once after the row sum.
 * y64[r] = s[r] * sum (fp64); y[r] = that value rounded to fp32. A field with
 * both bits set has no meaning on the page: it is rejected (OR_EINVAL). */
int or_ternary_gemv(const uint32_t* packed, const float* row_scale, const float* x,
                    float* y, double* y64, int64_t n, int64_t k) {
    if (n < 0 || k < 0 || k % 16 != 0) return OR_EINVAL;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t r = 0; r < n; ++r) {
        const uint32_t* row = packed + r * (k / 16);
        double acc = 0.0;
        for (int64_t c = 0; c < k; ++c) {
            uint32_t word = row[c / 16];
            int j = (int)(c % 16);
            int plus = (int)((word >> (2 * j + 1)) & 1u);
            int minus = (int)((word >> (2 * j)) & 1u);
            if (plus && minus) bad = 1;
            else if (plus) acc += (double)x[c];
            else if (minus) acc -= (double)x[c];
        }
        double v = (double)row_scale[r] * acc;
        if (y64) y64[r] = v;
        if (y) y[r] = (float)v;
    }
    return bad ? OR_EINVAL : OR_OK;
}

/* Small-batch ternary GEMM: the ternary GEMV above applied to each of
 * `batch` rows of x ([FairyFuse] "总结与启示" names batched GEMM fusion for
 * speculative decoding as the next step; the computation is the same row
 * sum per activation row): y[b][r] = s[r] * sum_c t(r, c) x[b][c], fp64 sum,
 * rounded to fp32 once. x is [batch, k], y is [batch, n]. */
int or_ternary_gemm(const uint32_t* packed, const float* row_scale, const float* x, float* y,
                    double* y64, int64_t batch, int64_t n, int64_t k) {
    if (batch < 0 || n < 0 || k < 0 || k % 16 != 0) return OR_EINVAL;
    int bad = 0;
    for (int64_t b = 0; b < batch; ++b) {
        int st = or_ternary_gemv(packed, row_scale, x + b * k, y ? y + b * n : NULL,
                                 y64 ? y64 + b * n : NULL, n, k);
        if (st != OR_OK) bad = 1;
    }
    return bad ? OR_EINVAL : OR_OK;
}

/* The ternary weight in field j of a packed word (the encoding above): +1, -1
 * or 0; a field with both bits set sets *bad and reads as 0. */
static int ternary_field(uint32_t word, int j, int* bad) {
    int plus = (int)((word >> (2 * j + 1)) & 1u);
    int minus = (int)((word >> (2 * j)) & 1u);
    if (plus && minus) {
        *bad = 1;
        return 0;
    }
    return plus - minus;
}

/* Widely-linear complex layer of [FairyFuse] "复杂值广泛线性层的融合核调度":
 * y = U x + W conj(x), with x complex [k] and U, W complex [n, k]. Reading of
 * the page: each of the four real parts U_re, U_im, W_re, W_im is a ternary
 * matrix in the packing of the ternary GEMV above and carries its own per-row
 * scale, as every ternary GEMV on the page does, so that
 *   U[r][c] = s_Ure[r] t_Ure[r][c] + i s_Uim[r] t_Uim[r][c]   (W likewise).
 * This is that definition written out: the complex entries of U and W are
 * formed, multiplied with x and with its conjugate, and summed, in fp64 complex
 * arithmetic (real and imaginary parts kept as two doubles). The page's eight
 * real sub-GEMVs are not used here; the tests check the decomposition against
 * this definition.
 *   packed: four pointers, U_re, U_im, W_re, W_im, each uint32 [n, k/16]
 *   scale:  fp32 [4, n] in the same order
 *   y_re/y_im: fp32 [n] (the fp64 values rounded once); y64_re/y64_im: fp64
 *   (either pair may be NULL). */
int or_ternary_wl_gemv(const uint32_t* const packed[4], const float* scale, const float* x_re,
                       const float* x_im, float* y_re, float* y_im, double* y64_re,
                       double* y64_im, int64_t n, int64_t k) {
    if (n < 0 || k < 0 || k % 16 != 0) return OR_EINVAL;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t r = 0; r < n; ++r) {
        const uint32_t* row[4];
        for (int m = 0; m < 4; ++m) row[m] = packed[m] + r * (k / 16);
        double acc_re = 0.0, acc_im = 0.0;
        for (int64_t c = 0; c < k; ++c) {
            int j = (int)(c % 16);
            double t[4];
            for (int m = 0; m < 4; ++m) t[m] = (double)ternary_field(row[m][c / 16], j, &bad);
            /* complex entries U[r][c] = a + ib and W[r][c] = p + iq */
            double a = (double)scale[0 * n + r] * t[0], b = (double)scale[1 * n + r] * t[1];
            double p = (double)scale[2 * n + r] * t[2], q = (double)scale[3 * n + r] * t[3];
            /* x = u + iv and its conjugate u - iv */
            double u = (double)x_re[c], v = (double)x_im[c];
            double cu = u, cv = -v;
            /* (a + ib)(u + iv) + (p + iq)(cu + i cv) */
            acc_re += (a * u - b * v) + (p * cu - q * cv);
            acc_im += (a * v + b * u) + (p * cv + q * cu);
        }
        if (y64_re) y64_re[r] = acc_re;
        if (y64_im) y64_im[r] = acc_im;
        if (y_re) y_re[r] = (float)acc_re;
        if (y_im) y_im[r] = (float)acc_im;
    }
    return bad ? OR_EINVAL : OR_OK;
}

/* --------------------------------------------------------------- NVFP4 --- */

/* One NVFP4 element in the order of [SGLang-34222] "关键源码片段"
 * (modelopt_quant.py embedding()): the E2M1 value with its sign (code 8 is
 * -0.0), the block scale decoded from E4M3 to float, eff = float(scale *
 * global) in fp32, value * eff in fp32, then a round-to-nearest-even cast to
 * bf16. */
uint16_t or_nvfp4_element(int code, uint8_t block_scale, float global_scale) {
    float mag = (float)E2M1_MAGNITUDE[code & 7];
    float v = (code & 8) ? -mag : mag;
    float bs = (float)or_e4m3_to_double(block_scale);
    float eff = bs * global_scale;
    float p = v * eff;
    return or_bf16_from_double((double)p);
}

/* Row gather + dequantise: table [vocab, hidden/2] packed codes, block_scale
 * [vocab, hidden/16] E4M3 bytes (group of 16 columns), out [ntok, hidden]
 * bf16 patterns. hidden must be a multiple of the group size (the page's
 * create_weights guard). Ids outside [0, vocab) give a zero row and count in
 * *bad_ids. */
int or_nvfp4_gather(const uint8_t* table, const uint8_t* block_scale, float global_scale,
                    const int64_t* ids, uint16_t* out, int64_t vocab, int64_t hidden,
                    int64_t ntok, int64_t* bad_ids) {
    if (vocab < 0 || hidden < 0 || ntok < 0 || hidden % 16 != 0) return OR_EINVAL;
    int64_t bad = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t t = 0; t < ntok; ++t) {
        int64_t id = ids[t];
        uint16_t* orow = out + t * hidden;
        if (id < 0 || id >= vocab) {
            for (int64_t c = 0; c < hidden; ++c) orow[c] = 0;
            bad += 1;
            continue;
        }
        const uint8_t* prow = table + id * (hidden / 2);
        const uint8_t* srow = block_scale + id * (hidden / 16);
        for (int64_t c = 0; c < hidden; ++c)
            orow[c] = or_nvfp4_element(code_at(prow, c), srow[c / 16], global_scale);
    }
    if (bad_ids) *bad_ids = bad;
    return OR_OK;
}

/* ----------------------------------------------------------- quantizers --- */

/* The pages use quantized weights but print no encoder: the MoE test of
 * [vLLM-51583] ("关键源码片段") calls an MXFP4 quantizer on bf16 weights and
 * shows only its outputs (codes [.., K/2], E8M0 scales [.., K/32]); the NVFP4
 * page ([SGLang-34222]) shows only the dequantisation. Reading taken (the
 * OCP microscaling rule for MXFP4, and the same element rounding for NVFP4):
 * an element is the E2M1 value nearest to its scaled input, ties to the code
 * whose last bit is 0, magnitudes above 6 saturate to 6, and the sign bit is
 * the input's (so a small negative input gives code 8). */
static int e2m1_encode(double v) {
    int sign = signbit(v) ? 8 : 0;
    double a = fabs(v);
    if (a >= 6.0) return sign | 7;
    int best = 0;
    double bd = a;
    for (int i = 1; i < 8; ++i) {
        double d = fabs(a - E2M1_MAGNITUDE[i]);
        if (d < bd || (d == bd && (i % 2) == 0)) {
            best = i;
            bd = d;
        }
    }
    return sign | best;
}

/* OCP E4M3 (e4m3fn) byte nearest to a non-negative value, ties to an even
 * mantissa, saturating at 448 (the format has no infinity; S.1111.111 is NaN). */
static uint8_t e4m3_encode(double t) {
    if (t >= 448.0) return 0x7E;
    uint8_t best = 0;
    double bd = t;
    for (int b = 1; b <= 0x7E; ++b) {
        double d = fabs(t - or_e4m3_to_double((uint8_t)b));
        if (d < bd || (d == bd && (b % 2) == 0)) {
            best = (uint8_t)b;
            bd = d;
        }
    }
    return best;
}

uint8_t or_e2m1_encode(double v) { return (uint8_t)e2m1_encode(v); }
uint8_t or_e4m3_encode(double t) { return e4m3_encode(t); }

/* MXFP4 quantizer for bf16 rows x [rows, k]: per 32 consecutive columns the
 * E8M0 exponent is floor(log2(amax)) - 2 (so that amax / 2^e lies in [4, 8),
 * the top binade of E2M1), biased by 127 and clamped to 0..254; an all-zero
 * block gets 0. Each element is then encoded from x / 2^(e - 127) (exact).
 * Codes pack as the decoder reads them (low nibble = even column). A
 * non-finite input is rejected (OR_EINVAL). */
int or_mxfp4_quantize(const uint16_t* x, uint8_t* packed, uint8_t* scales, int64_t rows, int64_t k) {
    if (rows < 0 || k < 0 || k % 32 != 0) return OR_EINVAL;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < k / 32; ++b) {
            const uint16_t* xb = x + r * k + 32 * b;
            double amax = 0.0;
            for (int i = 0; i < 32; ++i) {
                double v = or_double_from_bf16(xb[i]);
                if (!isfinite(v)) bad = 1;
                else if (fabs(v) > amax) amax = fabs(v);
            }
            int e = 0;
            if (amax > 0.0) {
                int ex;
                (void)frexp(amax, &ex);         /* amax in [2^(ex-1), 2^ex) */
                e = (ex - 1) - 2 + 127;
                if (e < 0) e = 0;
                if (e > 254) e = 254;
            }
            scales[r * (k / 32) + b] = (uint8_t)e;
            for (int i = 0; i < 32; i += 2) {
                int lo = e2m1_encode(ldexp(or_double_from_bf16(xb[i]), 127 - e));
                int hi = e2m1_encode(ldexp(or_double_from_bf16(xb[i + 1]), 127 - e));
                packed[r * (k / 2) + 16 * b + i / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
    }
    return bad ? OR_EINVAL : OR_OK;
}

/* NVFP4 quantizer for bf16 rows x [rows, k] with a given fp32 global scale g
 * (the per-tensor factor of [SGLang-34222]): per 16 consecutive columns the
 * block scale is the E4M3 value nearest to fl32(amax / fl32(6 g)), so that the
 * block's largest element maps to about 6; the element decoded scale is
 * eff = fl32(e4m3(bs) * g) in the order the dequantisation of that page uses,
 * and each element is encoded from fl32(x / eff) (eff = 0 gives signed zero
 * codes). Every fp32 step is an IEEE fp32 operation, so that a GPU taking the
 * same steps takes the same decisions. Rejects non-finite inputs and g <= 0. */
int or_nvfp4_quantize(const uint16_t* x, float g, uint8_t* packed, uint8_t* block_scale, int64_t rows,
                      int64_t k) {
    if (rows < 0 || k < 0 || k % 16 != 0 || !(g > 0.0f) || !isfinite(g)) return OR_EINVAL;
    const float d = 6.0f * g;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < k / 16; ++b) {
            const uint16_t* xb = x + r * k + 16 * b;
            float amax = 0.0f;
            for (int i = 0; i < 16; ++i) {
                float v = (float)or_double_from_bf16(xb[i]);
                if (!isfinite(v)) bad = 1;
                else if (fabsf(v) > amax) amax = fabsf(v);
            }
            float t = amax / d;
            uint8_t bs = e4m3_encode((double)t);
            block_scale[r * (k / 16) + b] = bs;
            float eff = (float)or_e4m3_to_double(bs) * g;
            for (int i = 0; i < 16; i += 2) {
                int c[2];
                for (int h = 0; h < 2; ++h) {
                    float v = (float)or_double_from_bf16(xb[i + h]);
                    if (eff == 0.0f) c[h] = signbit(v) ? 8 : 0;
                    else {
                        float q = v / eff;
                        c[h] = e2m1_encode((double)q);
                    }
                }
                packed[r * (k / 2) + 8 * b + i / 2] = (uint8_t)(c[0] | (c[1] << 4));
            }
        }
    }
    return bad ? OR_EINVAL : OR_OK;
}

/* ------------------------------------------------------ N:M structured --- */

/* N:M structured sparsity of [NM-wiki] (sglang-jax wiki page on the N:M
 * structured sparse matmul gap), sections "N:M 稀疏原理" and "3.1 Sparsifier":
 * in every group of M consecutive columns of a row, N values are kept. The
 * encoder takes, per group, the N positions with the largest mask values
 * (ties to the lower position; with a 0/1 mask holding N ones these are its
 * ones, in increasing order), gathers the values there, and packs the
 * in-group positions with next_log2(M) bits each, 32 / bits per 32-bit word,
 * position i of the sequence at bit (i mod packing) * bits of word
 * i / packing. The page's listing is abridged (several arrays are undefined)
 * and does not fix the array layout; the reading taken is one row after the
 * other: values [rows, (k/M) N] (bf16 here), positions in the same order,
 * packed per row into ceil((k/M) N / packing) words. */
int or_nm_bits(int m) {
    int b = 0;
    while ((1 << b) < m) ++b;
    return b;
}

int or_nm_encode(const uint16_t* dense, const uint8_t* mask, uint16_t* values, uint32_t* meta, int64_t rows,
                 int64_t k, int nn, int mm) {
    if (rows < 0 || k < 0 || mm < 1 || mm > 16 || nn < 1 || nn > mm || k % mm != 0) return OR_EINVAL;
    const int bits = or_nm_bits(mm) > 0 ? or_nm_bits(mm) : 1;
    const int packing = 32 / bits;
    const int64_t per_row = (k / mm) * nn;
    const int64_t words = (per_row + packing - 1) / packing;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t w = 0; w < words; ++w) meta[r * words + w] = 0u;
        for (int64_t g = 0; g < k / mm; ++g) {
            const uint8_t* mg = mask + r * k + g * mm;
            int taken[16] = {0};
            int sel[16];
            for (int j = 0; j < nn; ++j) {   /* top-N of the mask, ties to the lower position */
                int best = -1;
                for (int i = 0; i < mm; ++i)
                    if (!taken[i] && (best < 0 || mg[i] > mg[best])) best = i;
                taken[best] = 1;
                sel[j] = best;
            }
            for (int a = 0; a < nn; ++a)     /* positions in increasing order */
                for (int b = a + 1; b < nn; ++b)
                    if (sel[b] < sel[a]) {
                        int tmp = sel[a];
                        sel[a] = sel[b];
                        sel[b] = tmp;
                    }
            for (int j = 0; j < nn; ++j) {
                const int64_t e = g * nn + j;
                values[r * per_row + e] = dense[r * k + g * mm + sel[j]];
                meta[r * words + e / packing] |= (uint32_t)sel[j] << ((e % packing) * bits);
            }
        }
    }
    return OR_OK;
}

/* Decode: scatter the values back to their columns of a zero matrix (bf16
 * patterns) and set the mask; a position repeated within a group is rejected. */
int or_nm_decode(const uint16_t* values, const uint32_t* meta, uint16_t* dense, uint8_t* mask, int64_t rows,
                 int64_t k, int nn, int mm) {
    if (rows < 0 || k < 0 || mm < 1 || mm > 16 || nn < 1 || nn > mm || k % mm != 0) return OR_EINVAL;
    const int bits = or_nm_bits(mm) > 0 ? or_nm_bits(mm) : 1;
    const int packing = 32 / bits;
    const int64_t per_row = (k / mm) * nn;
    const int64_t words = (per_row + packing - 1) / packing;
    int bad = 0;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t c = 0; c < k; ++c) {
            dense[r * k + c] = 0;
            mask[r * k + c] = 0;
        }
        for (int64_t e = 0; e < per_row; ++e) {
            const uint32_t pos = (meta[r * words + e / packing] >> ((e % packing) * bits)) & ((1u << bits) - 1u);
            const int64_t col = (e / nn) * mm + pos;
            if ((int)pos >= mm || mask[r * k + col]) bad = 1;
            else {
                dense[r * k + col] = values[r * per_row + e];
                mask[r * k + col] = 1;
            }
        }
    }
    return bad ? OR_EINVAL : OR_OK;
}

/* Sparse matmul of the same page ("3.2", decompress then a dense product):
 * y[b][r] = sum over the row's kept entries of value * x[b][column], fp64
 * sums of the bf16 values times bf16 x, rounded once to fp32. */
int or_nm_spmm(const uint16_t* values, const uint32_t* meta, const uint16_t* x, double* y64, int64_t batch,
               int64_t rows, int64_t k, int nn, int mm) {
    if (batch < 0 || rows < 0 || k < 0 || mm < 1 || mm > 16 || nn < 1 || nn > mm || k % mm != 0)
        return OR_EINVAL;
    const int bits = or_nm_bits(mm) > 0 ? or_nm_bits(mm) : 1;
    const int packing = 32 / bits;
    const int64_t per_row = (k / mm) * nn;
    const int64_t words = (per_row + packing - 1) / packing;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < batch; ++b) {
            double acc = 0.0;
            for (int64_t e = 0; e < per_row; ++e) {
                const uint32_t pos = (meta[r * words + e / packing] >> ((e % packing) * bits)) & ((1u << bits) - 1u);
                if ((int)pos >= mm) {
                    bad = 1;
                    continue;
                }
                const int64_t col = (e / nn) * mm + pos;
                acc += or_double_from_bf16(values[r * per_row + e]) * or_double_from_bf16(x[b * k + col]);
            }
            y64[b * rows + r] = acc;
        }
    }
    return bad ? OR_EINVAL : OR_OK;
}

/* ----------------------------------------------------------------- MoE --- */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* MXFP4 mixture-of-experts layer with routing given as input, the semantics
 * exercised by [vLLM-51583] "关键源码片段" (the MoE test calls the fused
 * expert op with top-k weights and ids; the first expert matrix has 2N rows
 * and the activation is silu(gate) * up). For token t and slot j, with
 * expert e = ids[t, j]:
 *   h = W13[e] x_t            (2*inter outputs; rows [0, inter) are gate,
 *                              rows [inter, 2*inter) are up)
 *   a = silu(h[:inter]) * h[inter:]
 *   y = W2[e] a               (hidden outputs)
 *   out64[t] = sum_j weights[t, j] * y     (slot order)
 * all in fp64. Weights: w13 [E, 2*inter, hidden/2] + w13s [E, 2*inter,
 * hidden/32]; w2 [E, hidden, inter/2] + w2s [E, hidden, inter/32].
 * Pairs are grouped by expert only so that each weight row is decoded once;
 * every dot product still runs over its columns in order. */
int or_mxfp4_moe(const uint16_t* x, const uint8_t* w13, const uint8_t* w13s,
                 const uint8_t* w2, const uint8_t* w2s, const int32_t* ids,
                 const float* weights, double* out64, int64_t tokens, int64_t hidden,
                 int64_t inter, int64_t experts, int64_t topk) {
    if (tokens < 0 || hidden <= 0 || inter <= 0 || experts <= 0 || topk < 0) return OR_EINVAL;
    if (hidden % 32 != 0 || inter % 32 != 0) return OR_EINVAL;
    int64_t npairs = tokens * topk;
    for (int64_t p = 0; p < npairs; ++p)
        if (ids[p] < 0 || ids[p] >= experts) return OR_EINVAL;

    double* xd = (double*)malloc(sizeof(double) * (size_t)(tokens * hidden + 1));
    double* h = (double*)malloc(sizeof(double) * (size_t)(npairs * 2 * inter + 1));
    double* act = (double*)malloc(sizeof(double) * (size_t)(npairs * inter + 1));
    double* y = (double*)malloc(sizeof(double) * (size_t)(npairs * hidden + 1));
    int64_t* members = (int64_t*)malloc(sizeof(int64_t) * (size_t)(npairs + 1));
    if (!xd || !h || !act || !y || !members) {
        free(xd); free(h); free(act); free(y); free(members);
        return OR_ENOMEM;
    }
    for (int64_t i = 0; i < tokens * hidden; ++i) xd[i] = or_double_from_bf16(x[i]);

    int fail = 0;
    for (int64_t e = 0; e < experts; ++e) {
        int64_t m = 0;
        for (int64_t p = 0; p < npairs; ++p)
            if (ids[p] == e) members[m++] = p;
        if (m == 0) continue;
        const uint8_t* we13 = w13 + e * (2 * inter) * (hidden / 2);
        const uint8_t* se13 = w13s + e * (2 * inter) * (hidden / 32);
        const uint8_t* we2 = w2 + e * hidden * (inter / 2);
        const uint8_t* se2 = w2s + e * hidden * (inter / 32);
#pragma omp parallel reduction(| : fail)
        {
            int64_t len = hidden > inter ? hidden : inter;
            double* w = (double*)malloc(sizeof(double) * (size_t)len);
            if (!w) {
                fail = 1;
            } else {
                /* h = W13[e] x_t for every pair routed to e */
#pragma omp for schedule(static)
                for (int64_t r = 0; r < 2 * inter; ++r) {
                    const uint8_t* prow = we13 + r * (hidden / 2);
                    const uint8_t* srow = se13 + r * (hidden / 32);
                    for (int64_t c = 0; c < hidden; ++c) w[c] = mxfp4_value(code_at(prow, c), srow[c / 32]);
                    for (int64_t i = 0; i < m; ++i) {
                        int64_t p = members[i];
                        const double* xt = xd + (p / topk) * hidden;
                        double acc = 0.0;
                        for (int64_t c = 0; c < hidden; ++c) acc += w[c] * xt[c];
                        h[p * 2 * inter + r] = acc;
                    }
                }
                /* a = silu(gate) * up */
#pragma omp for schedule(static)
                for (int64_t i = 0; i < m; ++i) {
                    int64_t p = members[i];
                    for (int64_t c = 0; c < inter; ++c)
                        act[p * inter + c] = silu(h[p * 2 * inter + c]) * h[p * 2 * inter + inter + c];
                }
                /* y = W2[e] a */
#pragma omp for schedule(static)
                for (int64_t r = 0; r < hidden; ++r) {
                    const uint8_t* prow = we2 + r * (inter / 2);
                    const uint8_t* srow = se2 + r * (inter / 32);
                    for (int64_t c = 0; c < inter; ++c) w[c] = mxfp4_value(code_at(prow, c), srow[c / 32]);
                    for (int64_t i = 0; i < m; ++i) {
                        int64_t p = members[i];
                        const double* a = act + p * inter;
                        double acc = 0.0;
                        for (int64_t c = 0; c < inter; ++c) acc += w[c] * a[c];
                        y[p * hidden + r] = acc;
                    }
                }
                free(w);
            }
        }
    }
    /* weighted combine, slot order */
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < tokens; ++t)
        for (int64_t c = 0; c < hidden; ++c) {
            double acc = 0.0;
            for (int64_t j = 0; j < topk; ++j)
                acc += (double)weights[t * topk + j] * y[(t * topk + j) * hidden + c];
            out64[t * hidden + c] = acc;
        }
    free(xd); free(h); free(act); free(y); free(members);
    return fail ? OR_ENOMEM : OR_OK;
}
