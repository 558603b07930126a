/*
 * CPU oracle for the small-M BF16 x NVFP4 (W4A16) GEMV and its variants.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no code, header, table or helper with
 * the HIP library.
 *
 * Plain, slow and written to be checked by eye against the pages it follows:
 *   [gemv]   vllm.models.flint.ops.nvfp4_gemv   (module docstring "Numerics",
 *            nvfp4_gemv / bf16_gemv / dequantize_rows docstrings)
 *   [linear] vllm.models.flint.ops.linear        (_swizzled_scale_buffer,
 *            _dequant_gemm docstrings)
 *   [moe]    vllm.models.flint.ops.moe_gemv      (module docstring,
 *            gate_up / down_combine docstrings)
 * Every floating-point step is carried out in IEEE binary64 and each BF16
 * result is rounded exactly once, directly from the binary64 value
 * (round to nearest, ties to even).  Sums run over k in ascending order.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - E2M1 values: the OCP Microscaling (MX) v1.0 FP4 E2M1 element format
 *     (bias 1, one mantissa bit, no inf/NaN); the pages only name the codes.
 *   - E4M3 values: torch.float8_e4m3fn, i.e. OCP E4M3FN (bias 7, no inf,
 *     NaN at 0x7F/0xFF, largest finite 448).
 *   - 128x4 swizzle: the pages give only its name and byte size; the layout
 *     is the 128-row x 4-column block-scale tile layout of NVIDIA's public
 *     cuBLAS / PTX documentation (see oracle_scale_offset).
 *   - Final rounding mode: round to nearest, ties to even.
 *   - Routed experts use the same ModelOpt [gate; up] weight layout and flat
 *     128x4 scales as the shared expert; routed SiLU is the exact SiLU.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads used by the loops over independent outputs (rows n, pairs p).
 * Splitting the loop over outputs changes no arithmetic. */
int oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* Element formats                                                     */
/* ------------------------------------------------------------------ */

/* FP4 E2M1 code -> value.  [gemv] module docstring: the weight holds "E2M1
 * codes".  Code bits: sign (bit 3), exponent (bits 2..1, bias 1), mantissa
 * (bit 0); exponent 0 is subnormal (0 or 0.5).  Code 8 is -0. */
double oracle_e2m1_value(int code)
{
    int sign = (code >> 3) & 1;
    int exponent = (code >> 1) & 3;
    int mantissa = code & 1;
    double magnitude;
    if (exponent == 0)
        magnitude = 0.5 * mantissa;
    else
        magnitude = ldexp(1.0 + 0.5 * mantissa, exponent - 1);
    return sign ? -magnitude : magnitude;
}

/* FP8 E4M3FN byte -> value (torch.float8_e4m3fn, the scale dtype named in
 * [gemv] dequantize_rows and [linear] _swizzled_scale_buffer).  Bits: sign
 * (7), exponent (6..3, bias 7), mantissa (2..0).  Exponent 15 with
 * mantissa 7 is NaN; there is no infinity. */
double oracle_e4m3_value(int byte)
{
    int sign = (byte >> 7) & 1;
    int exponent = (byte >> 3) & 15;
    int mantissa = byte & 7;
    double magnitude;
    if (exponent == 15 && mantissa == 7)
        return NAN;
    if (exponent == 0)
        magnitude = ldexp(mantissa / 8.0, -6);
    else
        magnitude = ldexp(1.0 + mantissa / 8.0, exponent - 7);
    return sign ? -magnitude : magnitude;
}

/* BF16 bit pattern -> value. */
double oracle_bf16_to_f64(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* binary64 -> BF16, round to nearest, ties to even, in ONE step (no
 * intermediate binary32 rounding).  Overflow goes to +-inf, NaN to the
 * quiet NaN 0x7FC0 with the input's sign. */
uint16_t oracle_bf16_from_f64(double v)
{
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (isnan(v))
        return (uint16_t)(sign | 0x7FC0u);
    if (a == 0.0)
        return sign;
    /* a = f * 2^e with f in [0.5, 1): the leading bit has weight 2^(e-1). */
    int e;
    frexp(a, &e);
    int lead = e - 1;
    if (lead < -126)
        lead = -126;                         /* subnormal spacing 2^-133 */
    double ulp = ldexp(1.0, lead - 7);       /* 8 significant bits */
    double q = a / ulp;                      /* exact: power-of-two scaling */
    double fl = floor(q);
    double frac = q - fl;
    double r;
    if (frac > 0.5)
        r = fl + 1.0;
    else if (frac < 0.5)
        r = fl;
    else
        r = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
    double rounded = r * ulp;
    if (rounded > ldexp(255.0, 120))         /* largest finite BF16 = 0x7F7F */
        return (uint16_t)(sign | 0x7F80u);
    float f = (float)rounded;                /* exact: a BF16 value */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | ((u >> 16) & 0x7FFFu));
}

/* ------------------------------------------------------------------ */
/* 128x4-swizzled scale layout                                         */
/* ------------------------------------------------------------------ */

/* Number of scale columns after padding to a multiple of 4 (the "x4"). */
static int64_t padded_scale_cols(int64_t K)
{
    return ((K / 16) + 3) / 4 * 4;
}

/* Byte size of the flat buffer: [linear] _swizzled_scale_buffer computes it
 * as rows rounded up to 128 times scale columns rounded up to 4. */
int64_t oracle_scale_bytes(int64_t N, int64_t K)
{
    return (N + 127) / 128 * 128 * padded_scale_cols(K);
}

/* Offset of the scale of row n, scale column c (= k / 16) in the flat
 * buffer.  The buffer is a sequence of 512-byte tiles, each holding 128 rows
 * x 4 columns; tiles are ordered by 128-row band, then by 4-column group.
 * Inside a tile, row r sits in the 16-byte chunk r % 32, at 4-byte slot
 * r / 32, and the column within the group is the byte inside that slot. */
int64_t oracle_scale_offset(int64_t n, int64_t c, int64_t K)
{
    int64_t col_groups = padded_scale_cols(K) / 4;
    int64_t band = n / 128;
    int64_t r = n % 128;
    int64_t tile = band * col_groups + c / 4;
    return tile * 512 + (r % 32) * 16 + (r / 32) * 4 + (c % 4);
}

/* Logical [N][K/16] scales -> flat swizzled buffer; padding bytes are 0. */
void oracle_swizzle_scales(const uint8_t *logical, int64_t N, int64_t K, uint8_t *flat)
{
    int64_t cols = K / 16;
    memset(flat, 0, (size_t)oracle_scale_bytes(N, K));
    for (int64_t n = 0; n < N; ++n)
        for (int64_t c = 0; c < cols; ++c)
            flat[oracle_scale_offset(n, c, K)] = logical[n * cols + c];
}

/* Flat swizzled buffer -> logical [N][K/16] scales. */
void oracle_unswizzle_scales(const uint8_t *flat, int64_t N, int64_t K, uint8_t *logical)
{
    int64_t cols = K / 16;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t c = 0; c < cols; ++c)
            logical[n * cols + c] = flat[oracle_scale_offset(n, c, K)];
}

/* ------------------------------------------------------------------ */
/* Exact dequantization                                                */
/* ------------------------------------------------------------------ */

/* E2M1 code of weight (n, k): two codes per byte, the LOW nibble holds the
 * even k ([gemv] module docstring: "low nibble first"). */
static int weight_code(const uint8_t *w, int64_t K, int64_t n, int64_t k)
{
    uint8_t byte = w[n * (K / 2) + k / 2];
    return (k % 2 == 0) ? (byte & 15) : (byte >> 4);
}

/* One dequantized weight as a binary64 value: e2m1 * e4m3 with the scale of
 * the 16-weight block k / 16.  *inexact is set when the product is not a
 * BF16 value (the pages state that it always is for finite scales). */
static double dequant_weight(const uint8_t *w, const uint8_t *s_flat, int64_t K,
                             int64_t n, int64_t k, int *inexact)
{
    double scale = oracle_e4m3_value(s_flat[oracle_scale_offset(n, k / 16, K)]);
    double v = oracle_e2m1_value(weight_code(w, K, n, k)) * scale;
    if (!isnan(v) && oracle_bf16_to_f64(oracle_bf16_from_f64(v)) != v)
        *inexact = 1;
    return v;
}

/* [gemv] dequantize_rows: the exact BF16 e2m1 * e4m3 of every weight row
 * (global scale not applied).  Returns the number of products that were not
 * exactly representable in BF16 (0 for every finite scale). */
int64_t oracle_dequantize_rows(const uint8_t *w, const uint8_t *s_flat, int64_t rows,
                               int64_t K, uint16_t *out)
{
    int64_t not_exact = 0;
    for (int64_t n = 0; n < rows; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int inexact = 0;
            double v = dequant_weight(w, s_flat, K, n, k, &inexact);
            not_exact += inexact;
            out[n * K + k] = oracle_bf16_from_f64(v);
        }
    return not_exact;
}

/* ------------------------------------------------------------------ */
/* Dense GEMV                                                          */
/* ------------------------------------------------------------------ */

static double silu(double g)
{
    return g / (1.0 + exp(-g));
}

/* Row n of the dequantized weight into dst[K] (binary64). */
static void dequant_row_nvfp4(const uint8_t *w, const uint8_t *s_flat, int64_t K,
                              int64_t n, double *dst)
{
    int ignored = 0;
    for (int64_t k = 0; k < K; ++k)
        dst[k] = dequant_weight(w, s_flat, K, n, k, &ignored);
}

static void row_bf16(const uint16_t *w, int64_t K, int64_t n, double *dst)
{
    for (int64_t k = 0; k < K; ++k)
        dst[k] = oracle_bf16_to_f64(w[n * K + k]);
}

/* acc = sum_k x[m][k] * row[k] and its magnitude sum_k |x[m][k] * row[k]|. */
static void dot_row(const uint16_t *x, int64_t ldx, int64_t m, int64_t K, const double *row,
                    double *acc, double *absacc)
{
    double a = 0.0, b = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double p = oracle_bf16_to_f64(x[m * ldx + k]) * row[k];
        a += p;
        b += fabs(p);
    }
    *acc = a;
    *absacc = b;
}

/* Shared body of the dense GEMVs.  w_nvfp4 != NULL selects NVFP4 weights
 * (with s_flat), otherwise w_bf16 holds BF16 [N][K] weights.
 *   out[m][n] = bf16(acc[m][n] * gs)                      (silu_mul == 0)
 *   out[m][j] = bf16(silu(g) * u), g = bf16(acc[m][j] * gs),
 *               u = bf16(acc[m][j + N/2] * gs)            (silu_mul != 0)
 * acc_out / abs_out (optional, [M][N]) receive the unscaled binary64
 * accumulator and sum |x*w| of every row, for error bounds. */
static void dense_gemv(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                       const uint8_t *w_nvfp4, const uint8_t *s_flat, const uint16_t *w_bf16,
                       double gs, int64_t N, int silu_mul, uint16_t *out,
                       double *acc_out, double *abs_out)
{
    double *acc = (double *)malloc(sizeof(double) * (size_t)(M * N));
    double *absacc = (double *)malloc(sizeof(double) * (size_t)(M * N));
#pragma omp parallel
    {
        double *row = (double *)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            if (w_nvfp4)
                dequant_row_nvfp4(w_nvfp4, s_flat, K, n, row);
            else
                row_bf16(w_bf16, K, n, row);
            for (int64_t m = 0; m < M; ++m)
                dot_row(x, ldx, m, K, row, &acc[m * N + n], &absacc[m * N + n]);
        }
        free(row);
    }
    if (!silu_mul) {
        for (int64_t m = 0; m < M; ++m)
            for (int64_t n = 0; n < N; ++n)
                out[m * N + n] = oracle_bf16_from_f64(acc[m * N + n] * gs);
    } else {
        int64_t half = N / 2;
        for (int64_t m = 0; m < M; ++m)
            for (int64_t j = 0; j < half; ++j) {
                double g = oracle_bf16_to_f64(oracle_bf16_from_f64(acc[m * N + j] * gs));
                double u = oracle_bf16_to_f64(oracle_bf16_from_f64(acc[m * N + half + j] * gs));
                out[m * half + j] = oracle_bf16_from_f64(silu(g) * u);
            }
    }
    if (acc_out)
        memcpy(acc_out, acc, sizeof(double) * (size_t)(M * N));
    if (abs_out)
        memcpy(abs_out, absacc, sizeof(double) * (size_t)(M * N));
    free(acc);
    free(absacc);
}

/* [gemv] nvfp4_gemv: out = bf16(fp32(x @ dequant(W)^T) * global_scale); with
 * silu_mul the output is silu(gate) * up of the BF16 [gate | up] halves. */
void oracle_nvfp4_gemv(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                       const uint8_t *w, const uint8_t *s_flat, float global_scale,
                       int64_t N, int silu_mul, uint16_t *out,
                       double *acc_out, double *abs_out)
{
    dense_gemv(x, M, K, ldx, w, s_flat, NULL, (double)global_scale, N, silu_mul, out,
               acc_out, abs_out);
}

/* [gemv] bf16_gemv: the same computation with a row-major BF16 [N][K]
 * weight and a global scale of one. */
void oracle_bf16_gemv(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                      const uint16_t *w, int64_t N, int silu_mul, uint16_t *out,
                      double *acc_out, double *abs_out)
{
    dense_gemv(x, M, K, ldx, NULL, NULL, w, 1.0, N, silu_mul, out, acc_out, abs_out);
}

/* ------------------------------------------------------------------ */
/* MoE decode pair                                                     */
/* ------------------------------------------------------------------ */

/* [moe] gate_up.  Routed: for each pair p = t * topk + j with expert
 * e = ids[p], act[p][i] = bf16(silu(g) * u) where g and u are the unrounded
 * accumulators of rows i and I + i of W1[e] times alpha[e].
 * Shared expert: sact[t][i] = bf16(silu(bf16(g)) * bf16(u)) with the
 * accumulators of Wsh scaled by gssh (rows i and SI + i).
 * Weights: w1 [E][2I][H/2], w1_sf E consecutive flat buffers of
 * oracle_scale_bytes(2I, H) bytes; wsh [2SI][H/2] with ssh flat.
 * acc_r / abs_r ([M*topk][2I]) and acc_s / abs_s ([M][2SI]) are optional. */
void oracle_moe_gate_up(const uint16_t *x, int64_t M, int64_t H, const int32_t *ids,
                        int64_t topk, const uint8_t *w1, const uint8_t *w1_sf,
                        const float *alpha, int64_t I, uint16_t *act,
                        const uint8_t *wsh, const uint8_t *ssh, const float *gssh,
                        int64_t SI, uint16_t *sact,
                        double *acc_r, double *abs_r, double *acc_s, double *abs_s)
{
    int64_t P = M * topk;
    int64_t w1_expert_bytes = 2 * I * (H / 2);
    int64_t s1_expert_bytes = oracle_scale_bytes(2 * I, H);
#pragma omp parallel
    {
        double *row_g = (double *)malloc(sizeof(double) * (size_t)H);
        double *row_u = (double *)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(dynamic)
        for (int64_t p = 0; p < P; ++p) {
            int64_t t = p / topk;
            int64_t e = ids[p];
            const uint8_t *we = w1 + e * w1_expert_bytes;
            const uint8_t *se = w1_sf + e * s1_expert_bytes;
            for (int64_t i = 0; i < I; ++i) {
                double ag, bg, au, bu;
                dequant_row_nvfp4(we, se, H, i, row_g);
                dequant_row_nvfp4(we, se, H, I + i, row_u);
                dot_row(x, H, t, H, row_g, &ag, &bg);
                dot_row(x, H, t, H, row_u, &au, &bu);
                double g = ag * (double)alpha[e];
                double u = au * (double)alpha[e];
                act[p * I + i] = oracle_bf16_from_f64(silu(g) * u);
                if (acc_r) {
                    acc_r[p * 2 * I + i] = ag;
                    acc_r[p * 2 * I + I + i] = au;
                }
                if (abs_r) {
                    abs_r[p * 2 * I + i] = bg;
                    abs_r[p * 2 * I + I + i] = bu;
                }
            }
        }
        free(row_g);
        free(row_u);
    }
    /* Shared expert: the dense silu_mul GEMV of the shared weights. */
    dense_gemv(x, M, H, H, wsh, ssh, NULL, (double)gssh[0], 2 * SI, 1, sact, acc_s, abs_s);
}

/* [moe] down_combine.  For token t and output row h:
 *   y_j   = bf16(act[t*topk+j] . W2[e_j][h] * alpha2[e_j])
 *   s     = sum_j tw[t][j] * y_j              (binary64, j ascending)
 *   y_sh  = bf16(sact[t] . Wsd[h] * gssd)
 *   out   = bf16(bf16(s) + y_sh)
 * w2 [E][H][I/2] with E flat scale buffers of oracle_scale_bytes(H, I);
 * wsd [H][SI/2] with ssd flat.  acc_r / abs_r ([M][topk][H]) and
 * acc_s / abs_s ([M][H]) are optional. */
void oracle_moe_down_combine(const uint16_t *act, const int32_t *ids, const float *tw,
                             int64_t M, int64_t topk, const uint8_t *w2, const uint8_t *w2_sf,
                             const float *alpha2, int64_t H, int64_t I,
                             const uint16_t *sact, const uint8_t *wsd, const uint8_t *ssd,
                             const float *gssd, int64_t SI, uint16_t *out,
                             double *acc_r, double *abs_r, double *acc_s, double *abs_s)
{
    int64_t w2_expert_bytes = H * (I / 2);
    int64_t s2_expert_bytes = oracle_scale_bytes(H, I);
#pragma omp parallel
    {
        double *row = (double *)malloc(sizeof(double) * (size_t)(I > SI ? I : SI));
#pragma omp for schedule(dynamic)
        for (int64_t h = 0; h < H; ++h) {
            for (int64_t t = 0; t < M; ++t) {
                double s = 0.0;
                for (int64_t j = 0; j < topk; ++j) {
                    int64_t p = t * topk + j;
                    int64_t e = ids[p];
                    double a, b;
                    dequant_row_nvfp4(w2 + e * w2_expert_bytes, w2_sf + e * s2_expert_bytes, I, h, row);
                    dot_row(act, I, p, I, row, &a, &b);
                    double y = oracle_bf16_to_f64(oracle_bf16_from_f64(a * (double)alpha2[e]));
                    s += (double)tw[p] * y;
                    if (acc_r)
                        acc_r[(t * topk + j) * H + h] = a;
                    if (abs_r)
                        abs_r[(t * topk + j) * H + h] = b;
                }
                double a, b;
                dequant_row_nvfp4(wsd, ssd, SI, h, row);
                dot_row(sact, SI, t, SI, row, &a, &b);
                double ysh = oracle_bf16_to_f64(oracle_bf16_from_f64(a * (double)gssd[0]));
                double s_rounded = oracle_bf16_to_f64(oracle_bf16_from_f64(s));
                out[t * H + h] = oracle_bf16_from_f64(s_rounded + ysh);
                if (acc_s)
                    acc_s[t * H + h] = a;
                if (abs_s)
                    abs_s[t * H + h] = b;
            }
        }
        free(row);
    }
}
