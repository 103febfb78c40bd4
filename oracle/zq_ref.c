/*
 * zq_ref.c -- plain, slow CPU oracle for the W8A8 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library, and the HIP library never
 * calls it.
 *
 * Pages cited (title, then the section used):
 *   [ZQN]  "[2022 NeurIPS] ZeroQuant: Efficient and Affordable Post-Training
 *          Quantization for Large-Scale Transformers" (reading notes):
 *          group-wise weight quantization; token-wise activation quantization;
 *          the kernel-fusion flowcharts (LN/GeLU + Quantize, GeMM + DeQuantize).
 *   [T36]  "探秘Transformer系列之（36）--- 大模型量化方案":
 *          1.1 LLM.int8() "方案" and "混合精度分解" (outlier columns in FP16),
 *          1.1.2 "8位数据类型和量化" (absmax quantization to [-127,127]),
 *          1.1.2 "逐向量量化" (outer-product denormalisation of an int GEMM),
 *          1.2.2 "用于激活的按token量化" (dynamic per-token scales; scaling the
 *          INT32 accumulation before the FP16 write), 1.2.2 "用于权重矩阵的分组量化".
 *   [IQ]   "Integer Quantization: Deep Dive": "乘加单元" (accumulator initialised
 *          with the bias), "如何进行量化？" (x_int = clamp(round(x/s + z))),
 *          "量化模拟" (dequant s*(x_int - z)), "量化误差" (rounding error <= s/2).
 *   [SQ]   "SmoothQuant技术解析：大模型INT8量化的突破与实践": 2.1 (naive absmax
 *          quantizer, torch.round), 2.2 (Y = (X diag(s)^-1)(diag(s) W)),
 *          3.2 (offline: scale and quantize W; online: X diag(s)^-1, quantize).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - rounding is round-half-to-even (the SQ 2.1 quantizer uses torch.round);
 *   - the code range is symmetric [-127, 127], zero-point 0;
 *   - s = fl32(absmax / 127); q = clamp(rne(fl32(y / s)), -127, 127); an
 *     all-zero token or group gets s = 0 and all codes 0;
 *   - a weight group is G consecutive output rows by all K input columns;
 *   - LayerNorm is the textbook affine form with biased variance; GeLU is the
 *     exact erf form;
 *   - the bias is added in float after dequantization and before the
 *     optional GeLU epilogue;
 *   - the SmoothQuant factor is s_j = sqrt(max_m |LN(X)_mj| / max_n |W_nj|)
 *     with gamma = 1, beta = 0 for the statistics; s_j = 1 if either max is 0.
 *
 * Arithmetic: fp64 everywhere the pages do not fix a precision.  The two
 * places where float decides an integer (the code q and, through it, the
 * scale) are taken in fp32, the precision of the stored scale.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ZQREF_OK 0
#define ZQREF_ERR_ARG 1
#define ZQREF_ERR_OVERFLOW 2

#define PRE_NONE 0
#define PRE_LAYERNORM 1
#define PRE_GELU 2
#define ACT_NONE 0
#define ACT_GELU 1

/* Thread count of the OpenMP loops below (for timing the oracle on one core
 * or on all of them; results do not depend on it). */
void zqref_set_threads(int n)
{
    omp_set_num_threads(n > 0 ? n : 1);
}

int zqref_max_threads(void)
{
    return omp_get_max_threads();
}

/* ---- IEEE binary16 <-> binary32/64, written from the format definition ---- */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
float zqref_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);               /* subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);   /* (1 + f/1024) * 2^(e-15) */
    return (float)(sign ? -v : v);                /* exact: fits in binary32 */
}

/* One correctly rounded (nearest, ties to even) conversion from binary64. */
uint16_t zqref_f64_to_f16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v))
        return 0x7e00;
    if (a >= 65520.0)                 /* halfway between 65504 and 2^16 rounds up */
        return sign | 0x7c00;
    if (a < ldexp(1.0, -14)) {        /* subnormal range: multiples of 2^-24 */
        double q = nearbyint(ldexp(a, 24));   /* exact scaling, one rounding */
        return sign | (uint16_t)q;            /* q == 1024 encodes 2^-14 */
    }
    int e;
    frexp(a, &e);                     /* a = m * 2^e, m in [0.5, 1) */
    e -= 1;                           /* a = m' * 2^e, m' in [1, 2) */
    double q = nearbyint(ldexp(a, 10 - e));   /* 11-bit significand, in [1024, 2048] */
    if (q >= 2048.0) {
        q = 1024.0;
        e += 1;
    }
    if (e > 15)
        return sign | 0x7c00;
    return sign | (uint16_t)(((e + 15) << 10) | ((int)q - 1024));
}

static double load_x(const void *X, int x_is_f16, int64_t idx)
{
    if (x_is_f16)
        return (double)zqref_f16_to_f32(((const uint16_t *)X)[idx]);
    return (double)((const float *)X)[idx];
}

/* Exact-erf GeLU in fp64: 0.5 x (1 + erf(x / sqrt 2)). */
static double gelu64(double x)
{
    return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));
}

/* ---- Step: the elementwise / reduction op that precedes quantization ---- */

/*
 * [ZQN] kernel-fusion flowchart: LN/GeLU runs before Quantize.
 * LayerNorm: mean and biased variance in fp64 (two passes), then
 * y_k = fl32((x_k - mu) * r * gamma_k + beta_k) with r = 1/sqrt(var + eps).
 * GeLU: y_k = fl32(gelu(x_k)).  NONE: y_k = x_k.
 * gamma/beta NULL mean 1 and 0.
 */
int zqref_preop(const void *X, int x_is_f16, int64_t M, int64_t K, int pre,
                const float *gamma, const float *beta, float eps, float *Y)
{
    if (!X || !Y || M < 0 || K < 1)
        return ZQREF_ERR_ARG;
    if (pre != PRE_NONE && pre != PRE_LAYERNORM && pre != PRE_GELU)
        return ZQREF_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++) {
        const int64_t row = m * K;
        if (pre == PRE_LAYERNORM) {
            double sum = 0.0;
            for (int64_t k = 0; k < K; k++)
                sum += load_x(X, x_is_f16, row + k);
            double mu = sum / (double)K;
            double ss = 0.0;
            for (int64_t k = 0; k < K; k++) {
                double d = load_x(X, x_is_f16, row + k) - mu;
                ss += d * d;
            }
            double var = ss / (double)K;
            double r = 1.0 / sqrt(var + (double)eps);
            for (int64_t k = 0; k < K; k++) {
                double g = gamma ? (double)gamma[k] : 1.0;
                double b = beta ? (double)beta[k] : 0.0;
                Y[row + k] = (float)((load_x(X, x_is_f16, row + k) - mu) * r * g + b);
            }
        } else if (pre == PRE_GELU) {
            for (int64_t k = 0; k < K; k++)
                Y[row + k] = (float)gelu64(load_x(X, x_is_f16, row + k));
        } else {
            for (int64_t k = 0; k < K; k++)
                Y[row + k] = (float)load_x(X, x_is_f16, row + k);
        }
    }
    return ZQREF_OK;
}

/* ---- Step: symmetric absmax quantization of one vector ---- */

/*
 * [T36] 1.1.2 absmax quantization; [IQ] "如何进行量化？" with z = 0.
 * a = max |v|; s = fl32(a / 127); q = clamp(rne(fl32(v / s)), -127, 127).
 * Returns s.  a = 0 gives s = 0 and all-zero codes.
 */
static float absmax_quantize(const float *v, int64_t n, int8_t *q)
{
    float a = 0.0f;
    for (int64_t i = 0; i < n; i++) {
        float t = fabsf(v[i]);
        if (t > a)
            a = t;
    }
    float s = a / 127.0f;
    for (int64_t i = 0; i < n; i++) {
        if (s == 0.0f) {
            q[i] = 0;
            continue;
        }
        float t = v[i] / s;                  /* fp32 division, correctly rounded */
        float r = nearbyintf(t);             /* ties to even (default mode) */
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        q[i] = (int8_t)r;
    }
    return s;
}

/* The unfused flowchart of the ZeroQuant reading notes (kernel-fusion figure,
 * before fusion): the LN/GeLU output is written to memory as FP16 and a
 * separate step reads it back and quantizes it.  Each fp32 value is rounded
 * once to binary16 (nearest, ties to even) and widened back, exactly. */
int zqref_round_to_f16(const float *Y, int64_t n, float *out)
{
    if ((!Y || !out) && n > 0)
        return ZQREF_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = zqref_f16_to_f32(zqref_f64_to_f16((double)Y[i]));
    return ZQREF_OK;
}

/* Quantize each row of Y [M x K] with its own scale (dynamic per-token). */
int zqref_quantize_rows(const float *Y, int64_t M, int64_t K, int8_t *Xq, float *s_x)
{
    if (!Y || !Xq || !s_x || M < 0 || K < 1)
        return ZQREF_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++)
        s_x[m] = absmax_quantize(Y + m * K, K, Xq + m * K);
    return ZQREF_OK;
}

/*
 * The fused prologue's result: y = preop(x), then per-token quantization
 * ([T36] 1.2.2 token-wise activation quantization; [ZQN] fused LN/GeLU +
 * Quantize).  Y_out (optional, [M x K] fp32) receives y.
 */
int zqref_prologue(const void *X, int x_is_f16, int64_t M, int64_t K, int pre,
                   const float *gamma, const float *beta, float eps,
                   int8_t *Xq, float *s_x, float *Y_out)
{
    if (!Xq || !s_x)
        return ZQREF_ERR_ARG;
    float *Y = Y_out ? Y_out : (float *)malloc(sizeof(float) * (size_t)(M * K > 0 ? M * K : 1));
    if (!Y)
        return ZQREF_ERR_ARG;
    int rc = zqref_preop(X, x_is_f16, M, K, pre, gamma, beta, eps, Y);
    if (rc == ZQREF_OK)
        rc = zqref_quantize_rows(Y, M, K, Xq, s_x);
    if (!Y_out)
        free(Y);
    return rc;
}

/* ---- Step: group-wise weight quantization (offline) ---- */

/*
 * [ZQN] group-wise quantization of W; [T36] 1.2.2 group-wise weight
 * quantization.  Group g = rows [g*G, (g+1)*G) by all K columns; one scale
 * per group, computed exactly as the per-token scale.
 */
int zqref_quantize_groups(const float *W, int64_t N, int64_t K, int64_t G,
                          int8_t *Wq, float *s_w)
{
    if (!W || !Wq || !s_w || N < 1 || K < 1 || G < 1 || N % G)
        return ZQREF_ERR_ARG;
    const int64_t ng = N / G;
#pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < ng; g++)
        s_w[g] = absmax_quantize(W + g * G * K, G * K, Wq + g * G * K);
    return ZQREF_OK;
}

/* ---- Step: SmoothQuant factors and the offline fold ---- */

/*
 * [SQ] 2.2 / 3.2: s is a per-input-channel vector; the activation side is
 * divided by s, the weight side multiplied by it.  The statistics use the
 * linear's actual input LN(X) with gamma = 1, beta = 0:
 *   a_j = max_m |LN(X)_mj|, w_j = max_n |W_nj|, s_j = fl32(sqrt(a_j / w_j)),
 * with s_j = 1 when a_j or w_j is 0.  (The square root is the even split of
 * the range between the two sides.)
 */
int zqref_smooth_factors(const void *X, int x_is_f16, int64_t M, int64_t K, float eps,
                         const float *W, int64_t N, float *s)
{
    if (!X || !W || !s || M < 1 || K < 1 || N < 1)
        return ZQREF_ERR_ARG;
    float *Y = (float *)malloc(sizeof(float) * (size_t)(M * K));
    if (!Y)
        return ZQREF_ERR_ARG;
    int rc = zqref_preop(X, x_is_f16, M, K, PRE_LAYERNORM, NULL, NULL, eps, Y);
    if (rc != ZQREF_OK) {
        free(Y);
        return rc;
    }
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < K; j++) {
        double a = 0.0, w = 0.0;
        for (int64_t m = 0; m < M; m++) {
            double t = fabs((double)Y[m * K + j]);
            if (t > a) a = t;
        }
        for (int64_t n = 0; n < N; n++) {
            double t = fabs((double)W[n * K + j]);
            if (t > w) w = t;
        }
        s[j] = (a > 0.0 && w > 0.0) ? (float)sqrt(a / w) : 1.0f;
    }
    free(Y);
    return ZQREF_OK;
}

/* LN(x; gamma/s, beta/s) = LN(x; gamma, beta) / s: the activation side of the fold. */
int zqref_fold_ln(const float *gamma, const float *beta, const float *s, int64_t K,
                  float *gamma_out, float *beta_out)
{
    if (!s || !gamma_out || !beta_out || K < 1)
        return ZQREF_ERR_ARG;
    for (int64_t j = 0; j < K; j++) {
        double g = gamma ? (double)gamma[j] : 1.0;
        double b = beta ? (double)beta[j] : 0.0;
        gamma_out[j] = (float)(g / (double)s[j]);
        beta_out[j] = (float)(b / (double)s[j]);
    }
    return ZQREF_OK;
}

/* W'_{n,j} = fl32(W_{n,j} * s_j): the weight side of the fold (columns of [N x K]). */
int zqref_fold_weights(const float *W, const float *s, int64_t N, int64_t K, float *W_out)
{
    if (!W || !s || !W_out || N < 1 || K < 1)
        return ZQREF_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++)
        for (int64_t j = 0; j < K; j++)
            W_out[n * K + j] = (float)((double)W[n * K + j] * (double)s[j]);
    return ZQREF_OK;
}

/* ---- Step: the integer GEMM ---- */

/*
 * [IQ] "乘加单元": each output accumulates products W_nm * x_m; [T36] 1.2.2:
 * the INT8 product accumulates in INT32.  acc[m,n] = sum_k Xq[m,k] * Wq[n,k],
 * exact in int64, then checked to fit int32.
 */
int zqref_gemm_i32(const int8_t *Xq, const int8_t *Wq, int64_t M, int64_t N, int64_t K,
                   int32_t *acc)
{
    if (!Xq || !Wq || !acc || M < 0 || N < 1 || K < 1)
        return ZQREF_ERR_ARG;
    int overflow = 0;
#pragma omp parallel for schedule(static) reduction(| : overflow)
    for (int64_t m = 0; m < M; m++) {
        for (int64_t n = 0; n < N; n++) {
            int64_t sum = 0;
            for (int64_t k = 0; k < K; k++)
                sum += (int64_t)Xq[m * K + k] * (int64_t)Wq[n * K + k];
            if (sum > INT32_MAX || sum < INT32_MIN)
                overflow = 1;
            acc[m * N + n] = (int32_t)sum;
        }
    }
    return overflow ? ZQREF_ERR_OVERFLOW : ZQREF_OK;
}

/* ---- Step: dequantization epilogue ---- */

/*
 * [T36] 1.1.2 vector-wise: the int product is denormalised by the outer
 * product of the row scales and the column scales; [T36] 1.2.2: the INT32
 * accumulation is scaled by the activation and weight scales before the
 * FP16 write; [IQ] "乘加单元": the bias joins the accumulation.
 *   v = s_x[m] * s_w[n / G] * acc[m,n] + b[n]   (fp64)
 *   v = gelu(v) if act == GELU                  (fp64)
 *   Y = fp16(v), one rounding, ties to even.
 * Y_f64 (optional) receives v before the fp16 rounding.
 */
int zqref_epilogue(const int32_t *acc, const float *s_x, const float *s_w, int64_t G,
                   const float *bias, int act, int64_t M, int64_t N,
                   uint16_t *Y, double *Y_f64)
{
    if (!acc || !s_x || !s_w || !Y || G < 1 || N % G || M < 0 || N < 1)
        return ZQREF_ERR_ARG;
    if (act != ACT_NONE && act != ACT_GELU)
        return ZQREF_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++) {
        for (int64_t n = 0; n < N; n++) {
            double v = (double)s_x[m] * (double)s_w[n / G] * (double)acc[m * N + n];
            if (bias)
                v += (double)bias[n];
            if (act == ACT_GELU)
                v = gelu64(v);
            if (Y_f64)
                Y_f64[m * N + n] = v;
            Y[m * N + n] = zqref_f64_to_f16(v);
        }
    }
    return ZQREF_OK;
}

/* ---- The FP8 variant ----
 *
 * [T36] 2 (ZeroQuant-FP): FP8 activations; every scale factor a power of
 * two, kept within one compute group.  Codes are the OCP 8-bit E4M3 format
 * (1 sign bit, 4 exponent bits with bias 7, 3 fraction bits; no infinities;
 * 0x7F and 0xFF are NaN; largest finite value 1.75 * 2^8 = 448; subnormals
 * f/8 * 2^-6).  Reading: the scale of a vector with absmax a > 0 is the
 * smallest power of two 2^e with a <= 448 * 2^e (nothing is clipped); a = 0
 * gives scale 0 and all codes 0.  A value y is coded as the E4M3 value
 * nearest to y / 2^e (an exact fp32 scaling), ties to even.
 */

double zqref_e4m3_to_f64(uint8_t c)
{
    const int sign = c >> 7, e = (c >> 3) & 15, f = c & 7;
    if (e == 15 && f == 7)
        return NAN;
    const double v = e == 0 ? ldexp((double)f, -9)          /* f/8 * 2^-6 */
                            : ldexp((double)(8 + f), e - 10); /* (1 + f/8) * 2^(e-7) */
    return sign ? -v : v;
}

/* Nearest E4M3 value, ties to even; |v| above 448 saturates to 448. */
uint8_t zqref_f64_to_e4m3(double v)
{
    const uint8_t sign = signbit(v) ? 0x80 : 0;
    const double a = fabs(v);
    if (isnan(v))
        return 0x7f;
    if (a >= 448.0)
        return sign | 0x7e;
    if (a < ldexp(1.0, -6)) {                      /* subnormal range: multiples of 2^-9 */
        const double q = nearbyint(ldexp(a, 9));   /* exact scaling, one rounding */
        return sign | (uint8_t)q;                  /* q == 8 encodes 2^-6 */
    }
    int e;
    frexp(a, &e);                                  /* a = m 2^e, m in [0.5, 1) */
    e -= 1;                                        /* a = m' 2^e, m' in [1, 2) */
    double q = nearbyint(ldexp(a, 3 - e));         /* 4-bit significand, in [8, 16] */
    if (q >= 16.0) {
        q = 8.0;
        e += 1;
    }
    if (e > 8 || (e == 8 && q > 14.0))             /* above 448 after rounding */
        return sign | 0x7e;
    return sign | (uint8_t)(((e + 7) << 3) | ((int)q - 8));
}

/* Smallest power of two 2^e with a <= 448 * 2^e (a > 0), else 0. */
float zqref_pow2_scale(float a)
{
    if (!(a > 0.0f))
        return 0.0f;
    int e;
    frexp((double)a, &e);          /* 2^(e-1) <= a < 2^e */
    e -= 8;                        /* 448 * 2^e >= 256 * 2^e ... start near the answer */
    while (448.0 * ldexp(1.0, e) < (double)a)
        e++;
    while (448.0 * ldexp(1.0, e - 1) >= (double)a)
        e--;
    return (float)ldexp(1.0, e);
}

static float pow2_quantize(const float *v, int64_t n, uint8_t *q)
{
    float a = 0.0f;
    for (int64_t i = 0; i < n; i++)
        a = fmaxf(a, fabsf(v[i]));
    const float s = zqref_pow2_scale(a);
    for (int64_t i = 0; i < n; i++)
        q[i] = s == 0.0f ? 0 : zqref_f64_to_e4m3((double)(v[i] / s));  /* exact division */
    return s;
}

/* Per-token FP8 codes of fp32 rows. */
int zqref_quantize_rows_fp8(const float *Y, int64_t M, int64_t K, uint8_t *q, float *s)
{
    if (!Y || !q || !s || M < 0 || K < 1)
        return ZQREF_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++)
        s[m] = pow2_quantize(Y + m * K, K, q + m * K);
    return ZQREF_OK;
}

/* Group-wise FP8 codes of weights: G consecutive output rows by all K columns. */
int zqref_quantize_groups_fp8(const float *W, int64_t N, int64_t K, int64_t G, uint8_t *q,
                              float *s)
{
    if (!W || !q || !s || N < 1 || K < 1 || G < 1 || N % G)
        return ZQREF_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < N / G; g++)
        s[g] = pow2_quantize(W + g * G * K, G * K, q + g * G * K);
    return ZQREF_OK;
}

/* acc[m,n] = sum_k dec(Xq[m,k]) dec(Wq[n,k]) in fp64 (each product is exact). */
int zqref_gemm_fp8(const uint8_t *Xq, const uint8_t *Wq, int64_t M, int64_t N, int64_t K,
                   double *acc)
{
    if (!Xq || !Wq || !acc || M < 0 || N < 1 || K < 1)
        return ZQREF_ERR_ARG;
    double lut[256];
    for (int c = 0; c < 256; c++)
        lut[c] = zqref_e4m3_to_f64((uint8_t)c);
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++) {
            double t = 0.0;
            for (int64_t k = 0; k < K; k++)
                t += lut[Xq[m * K + k]] * lut[Wq[n * K + k]];
            acc[m * N + n] = t;
        }
    return ZQREF_OK;
}

/* The dequantizing epilogue on fp64 accumulators (as zqref_epilogue). */
int zqref_epilogue_f64acc(const double *acc, const float *s_x, const float *s_w, int64_t G,
                          const float *bias, int act, int64_t M, int64_t N, uint16_t *Y)
{
    if (!acc || !s_x || !s_w || !Y || G < 1 || N % G || M < 0 || N < 1)
        return ZQREF_ERR_ARG;
    if (act != ACT_NONE && act != ACT_GELU)
        return ZQREF_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++) {
            double v = (double)s_x[m] * (double)s_w[n / G] * acc[m * N + n];
            if (bias)
                v += (double)bias[n];
            if (act == ACT_GELU)
                v = gelu64(v);
            Y[m * N + n] = zqref_f64_to_f16(v);
        }
    return ZQREF_OK;
}

/* ---- The whole layer on a subset of tokens ---- */

/*
 * The fused layer ([ZQN] flowchart after fusion: (LN/GeLU + Quantize) then
 * (GeMM + DeQuantize)) evaluated for the tokens listed in rows[0..R).
 * Each token is independent, so a subset gives exactly the rows of the full
 * result.  Outputs are [R x K] codes, [R] scales and [R x N] fp16.
 */
int zqref_linear_rows(const void *X, int x_is_f16, int64_t M, int64_t K, int pre,
                      const float *gamma, const float *beta, float eps,
                      const int8_t *Wq, const float *s_w, int64_t G, const float *bias,
                      int act, int64_t N, const int64_t *rows, int64_t R,
                      int8_t *Xq_out, float *s_x_out, uint16_t *Y_out)
{
    if (!X || !Wq || !s_w || !rows || !Xq_out || !s_x_out || !Y_out || R < 0)
        return ZQREF_ERR_ARG;
    for (int64_t r = 0; r < R; r++)
        if (rows[r] < 0 || rows[r] >= M)
            return ZQREF_ERR_ARG;
    const size_t esz = x_is_f16 ? 2 : 4;
    char *Xs = (char *)malloc(esz * (size_t)(R * K > 0 ? R * K : 1));
    int32_t *acc = (int32_t *)malloc(sizeof(int32_t) * (size_t)(R * N > 0 ? R * N : 1));
    if (!Xs || !acc) {
        free(Xs);
        free(acc);
        return ZQREF_ERR_ARG;
    }
    for (int64_t r = 0; r < R; r++)
        memcpy(Xs + esz * (size_t)(r * K), (const char *)X + esz * (size_t)(rows[r] * K), esz * (size_t)K);
    int rc = zqref_prologue(Xs, x_is_f16, R, K, pre, gamma, beta, eps, Xq_out, s_x_out, NULL);
    if (rc == ZQREF_OK)
        rc = zqref_gemm_i32(Xq_out, Wq, R, N, K, acc);
    if (rc == ZQREF_OK)
        rc = zqref_epilogue(acc, s_x_out, s_w, G, bias, act, R, N, Y_out, NULL);
    free(Xs);
    free(acc);
    return rc;
}

/*
 * The unquantized layer act(preop(X) W^T + b) in fp64, for a subset of
 * tokens.  Informational only (quantization error with and without the
 * SmoothQuant fold); it is not what the integer path is compared with.
 */
int zqref_linear_float_rows(const void *X, int x_is_f16, int64_t M, int64_t K, int pre,
                            const float *gamma, const float *beta, float eps,
                            const float *W, const float *bias, int act, int64_t N,
                            const int64_t *rows, int64_t R, double *Y_out)
{
    if (!X || !W || !rows || !Y_out || R < 0)
        return ZQREF_ERR_ARG;
    for (int64_t r = 0; r < R; r++)
        if (rows[r] < 0 || rows[r] >= M)
            return ZQREF_ERR_ARG;
    const size_t esz = x_is_f16 ? 2 : 4;
    char *Xs = (char *)malloc(esz * (size_t)(R * K > 0 ? R * K : 1));
    float *Y = (float *)malloc(sizeof(float) * (size_t)(R * K > 0 ? R * K : 1));
    if (!Xs || !Y) {
        free(Xs);
        free(Y);
        return ZQREF_ERR_ARG;
    }
    for (int64_t r = 0; r < R; r++)
        memcpy(Xs + esz * (size_t)(r * K), (const char *)X + esz * (size_t)(rows[r] * K), esz * (size_t)K);
    int rc = zqref_preop(Xs, x_is_f16, R, K, pre, gamma, beta, eps, Y);
    if (rc == ZQREF_OK) {
#pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < R; r++) {
            for (int64_t n = 0; n < N; n++) {
                double v = 0.0;
                for (int64_t k = 0; k < K; k++)
                    v += (double)Y[r * K + k] * (double)W[n * K + k];
                if (bias)
                    v += (double)bias[n];
                if (act == ACT_GELU)
                    v = gelu64(v);
                Y_out[r * N + n] = v;
            }
        }
    }
    free(Xs);
    free(Y);
    return rc;
}

/* ---- The LLM.int8() mixed-precision decomposition ----
 *
 * [T36] 1.1 LLM.int8(), "方案" and "混合精度分解": the matmul input is split
 * by column.  A column is an outlier dimension when some token's value there
 * exceeds the threshold alpha in magnitude (alpha = 6.0 is the page's
 * setting); the set O of such columns is found at run time over the whole
 * batch.  Columns in O are kept in FP16 on both sides and multiplied in high
 * precision (W16A16); the other columns are quantized vector-wise, each token
 * row with its own absmax, multiplied in INT8, and the INT32 product is
 * dequantized.  The two partial products are added into one FP16 result.
 *
 * Readings: "exceeds" is strict, |y| > alpha; the token absmax runs over the
 * columns outside O only, and the INT8 operand holds code 0 in the columns
 * of O; the INT8 weights are the layer's offline group-wise codes (G = 1 is
 * the page's per-output-channel scale), made over all K since O is not known
 * offline; the FP16 operands are fp16(y) and fp16(W), nearest with ties to
 * even; both partial products, the bias and the GeLU epilogue are summed in
 * fp64 and rounded to FP16 once.
 */

/* O = { j : max_m |Y[m, j]| > alpha }, ascending; *P = |O|. */
int zqref_outlier_columns(const float *Y, int64_t M, int64_t K, float alpha,
                          int32_t *cols, int64_t *P)
{
    if (!Y || !cols || !P || M < 0 || K < 1)
        return ZQREF_ERR_ARG;
    int64_t n = 0;
    for (int64_t j = 0; j < K; j++) {
        int hit = 0;
        for (int64_t m = 0; m < M && !hit; m++)
            hit = fabsf(Y[m * K + j]) > alpha;
        if (hit)
            cols[n++] = (int32_t)j;
    }
    *P = n;
    return ZQREF_OK;
}

/* Vector-wise quantization of each row of Y over the columns outside O:
 * a = max_{j not in O} |y_j|, s = fl32(a / 127), q_j as in absmax_quantize;
 * q_j = 0 for j in O. */
int zqref_quantize_rows_excluding(const float *Y, int64_t M, int64_t K, const int32_t *cols,
                                  int64_t P, int8_t *Xq, float *s_x)
{
    if (!Y || !Xq || !s_x || M < 0 || K < 1 || P < 0 || (P > 0 && !cols))
        return ZQREF_ERR_ARG;
    char *in_o = (char *)calloc((size_t)K, 1);
    if (!in_o)
        return ZQREF_ERR_ARG;
    for (int64_t p = 0; p < P; p++) {
        if (cols[p] < 0 || cols[p] >= K) {
            free(in_o);
            return ZQREF_ERR_ARG;
        }
        in_o[cols[p]] = 1;
    }
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++) {
        const float *y = Y + m * K;
        float a = 0.0f;
        for (int64_t j = 0; j < K; j++)
            if (!in_o[j] && fabsf(y[j]) > a)
                a = fabsf(y[j]);
        float s = a / 127.0f;
        s_x[m] = s;
        for (int64_t j = 0; j < K; j++) {
            if (in_o[j] || s == 0.0f) {
                Xq[m * K + j] = 0;
                continue;
            }
            float r = nearbyintf(y[j] / s);
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            Xq[m * K + j] = (int8_t)r;
        }
    }
    free(in_o);
    return ZQREF_OK;
}

/*
 * The decomposed epilogue: for token m and output n,
 *   v = s_x[m] s_w[n/G] acc[m,n] + sum_{p<P} fp16(Y[m, O_p]) fp16(W[n, O_p]) + b[n]
 * in fp64, then GeLU if asked, then one rounding to fp16.  Y is the op's
 * output [M x K] (fp32), W the unquantized weights [N x K] (fp32 or widened
 * fp16).  Y_f64 (optional) receives v before the rounding.
 */
int zqref_decomp_epilogue(const int32_t *acc, const float *s_x, const float *s_w, int64_t G,
                          const float *Y, int64_t K, const int32_t *cols, int64_t P,
                          const float *W, const float *bias, int act, int64_t M, int64_t N,
                          uint16_t *Yout, double *Y_f64)
{
    if (!acc || !s_x || !s_w || !Yout || G < 1 || N % G || M < 0 || N < 1 || K < 1 || P < 0)
        return ZQREF_ERR_ARG;
    if (P > 0 && (!Y || !W || !cols))
        return ZQREF_ERR_ARG;
    if (act != ACT_NONE && act != ACT_GELU)
        return ZQREF_ERR_ARG;
    for (int64_t p = 0; p < P; p++)
        if (cols[p] < 0 || cols[p] >= K)
            return ZQREF_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++) {
        for (int64_t n = 0; n < N; n++) {
            double v = (double)s_x[m] * (double)s_w[n / G] * (double)acc[m * N + n];
            for (int64_t p = 0; p < P; p++) {
                const int64_t j = cols[p];
                double a = (double)zqref_f16_to_f32(zqref_f64_to_f16((double)Y[m * K + j]));
                double w = (double)zqref_f16_to_f32(zqref_f64_to_f16((double)W[n * K + j]));
                v += a * w;
            }
            if (bias)
                v += (double)bias[n];
            if (act == ACT_GELU)
                v = gelu64(v);
            if (Y_f64)
                Y_f64[m * N + n] = v;
            Yout[m * N + n] = zqref_f64_to_f16(v);
        }
    }
    return ZQREF_OK;
}

/*
 * The decomposed layer for the tokens listed in rows[0..R).  The outlier set
 * depends on every token of the batch, so the op runs over all M tokens to
 * find O (cols[0..*P)); each listed token then follows the steps above.
 * Outputs: cols [K] (first *P used), Xq_out [R x K], s_x_out [R], Y_out [R x N].
 */
int zqref_linear_decomp_rows(const void *X, int x_is_f16, int64_t M, int64_t K, int pre,
                             const float *gamma, const float *beta, float eps, float alpha,
                             const int8_t *Wq, const float *s_w, int64_t G, const float *W,
                             const float *bias, int act, int64_t N, const int64_t *rows, int64_t R,
                             int32_t *cols, int64_t *P, int8_t *Xq_out, float *s_x_out,
                             uint16_t *Y_out)
{
    if (!X || !Wq || !s_w || !W || !rows || !cols || !P || !Xq_out || !s_x_out || !Y_out ||
        R < 0 || M < 1 || K < 1 || N < 1)
        return ZQREF_ERR_ARG;
    for (int64_t r = 0; r < R; r++)
        if (rows[r] < 0 || rows[r] >= M)
            return ZQREF_ERR_ARG;
    float *Y = (float *)malloc(sizeof(float) * (size_t)(M * K));
    float *Ys = (float *)malloc(sizeof(float) * (size_t)(R * K > 0 ? R * K : 1));
    int32_t *acc = (int32_t *)malloc(sizeof(int32_t) * (size_t)(R * N > 0 ? R * N : 1));
    int rc = ZQREF_ERR_ARG;
    if (Y && Ys && acc) {
        rc = zqref_preop(X, x_is_f16, M, K, pre, gamma, beta, eps, Y);
        if (rc == ZQREF_OK)
            rc = zqref_outlier_columns(Y, M, K, alpha, cols, P);
        if (rc == ZQREF_OK) {
            for (int64_t r = 0; r < R; r++)
                memcpy(Ys + r * K, Y + rows[r] * K, sizeof(float) * (size_t)K);
            rc = zqref_quantize_rows_excluding(Ys, R, K, cols, *P, Xq_out, s_x_out);
        }
        if (rc == ZQREF_OK)
            rc = zqref_gemm_i32(Xq_out, Wq, R, N, K, acc);
        if (rc == ZQREF_OK)
            rc = zqref_decomp_epilogue(acc, s_x_out, s_w, G, Ys, K, cols, *P, W, bias, act, R, N,
                                       Y_out, NULL);
    }
    free(Y);
    free(Ys);
    free(acc);
    return rc;
}
