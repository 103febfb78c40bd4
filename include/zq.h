/*
 * zq.h -- C ABI of libzq: ZeroQuant-style W8A8 inference for one linear layer
 * on AMD Instinct MI355X (gfx950).
 *
 * Pages cited (title, then section):
 *   [ZQN] "[2022 NeurIPS] ZeroQuant: Efficient and Affordable Post-Training
 *         Quantization for Large-Scale Transformers" (reading notes): group-wise
 *         weight quantization; token-wise activation quantization; the
 *         kernel-fusion flowcharts ("LN/GeLU + Quantize" then "GeMM + DeQuantize").
 *   [T36] "探秘Transformer系列之（36）--- 大模型量化方案": 1.1 LLM.int8() mixed-precision
 *         decomposition (outlier columns in FP16); 1.1.2 absmax quantization
 *         and vector-wise (outer-product) denormalisation; 1.2.2 token-wise
 *         activation quantization fused with the preceding LayerNorm, INT32
 *         accumulation scaled by both scales before the FP16 write, group-wise
 *         weight quantization; 1.3 granularity (scales only along the outer
 *         dimensions of an INT8 GEMM).
 *   [IQ]  "Integer Quantization: Deep Dive": MAC unit (accumulator plus bias);
 *         quantize / dequantize formulas with zero-point z = 0 here.
 *   [SQ]  "SmoothQuant技术解析：大模型INT8量化的突破与实践": 2.2 the smoothing
 *         identity Y = (X diag(s)^-1)(diag(s) W); 3.2 offline weight scaling and
 *         quantization, online activation division and quantization.
 *
 * Conventions for every call
 *   - Data pointers are DEVICE pointers owned by the caller; the library keeps
 *     no reference after the call returns and allocates no memory.
 *   - Work is enqueued asynchronously on `stream` (NULL = the default stream);
 *     results are ready when the stream is synchronised.
 *   - Matrices are row-major and dense: X [M x K], Xq [M x K], W / Wq [N x K]
 *     (output rows, input columns, so both GEMM operands are K-contiguous),
 *     Y [M x N].  M = tokens, K = input features, N = output features.
 *   - Size caps beyond each call's own rules: M, N <= 2^31 - 1 and every
 *     matrix a call reads or writes (M x K, N x K, M x N) has at most 2^40
 *     elements (the unfused layer caps M x N at 2^38, the FFN block M x F
 *     at 2^39, for their workspaces); larger sizes return ZQ_ERR_SHAPE, and
 *     the workspace-size helpers return 0.
 *   - Arguments are validated on the host before anything is enqueued; on an
 *     error nothing is enqueued and a non-zero zq_status is returned.  A
 *     launch failure reported by the HIP runtime returns ZQ_ERR_HIP.  Faults
 *     during execution surface at the caller's next synchronisation.
 *   - An error already pending on the calling thread when a call starts (left
 *     by the caller's earlier HIP work, as hipPeekAtLastError shows it) makes
 *     the call return ZQ_ERR_HIP before enqueueing anything; the error is left
 *     pending for the caller to read, never cleared by the library.
 *   - Calls never abort and never throw.  The library keeps no mutable global
 *     state: calls are reentrant; calls on different streams that write the
 *     same buffers race, as any two kernels would.
 *   - Quantization is symmetric absmax: s = fl32(max|v| / 127),
 *     q = clamp(round_half_even(fl32(v / s)), -127, 127), and an all-zero
 *     vector gets s = 0 with all codes 0 ([T36] 1.1.2; [IQ] with z = 0).
 */
#ifndef ZQ_H
#define ZQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum zq_status {
    ZQ_OK = 0,
    ZQ_ERR_NULL = 1,        /* a required pointer is NULL */
    ZQ_ERR_SHAPE = 2,       /* a size is out of range or not a required multiple */
    ZQ_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned */
    ZQ_ERR_DTYPE = 4,       /* a dtype / op enum is not one this argument accepts */
    ZQ_ERR_WORKSPACE = 5,   /* the workspace is NULL or smaller than required */
    ZQ_ERR_HIP = 6,         /* the HIP runtime reported an error at launch */
    ZQ_ERR_UNSUPPORTED = 7  /* a valid request the library does not implement */
} zq_status;

typedef enum zq_dtype {
    ZQ_F32 = 0,
    ZQ_F16 = 1,
    ZQ_I8 = 2,
    ZQ_I32 = 3
} zq_dtype;

/* The op fused in front of the per-token quantizer ([ZQN] flowchart). */
typedef enum zq_pre {
    ZQ_PRE_NONE = 0,
    ZQ_PRE_LAYERNORM = 1,   /* y = (x - mean) / sqrt(var + eps) * gamma + beta, biased var */
    ZQ_PRE_GELU = 2         /* y = x * Phi(x), the exact (erf) GeLU */
} zq_pre;

/* The op fused after the dequantization in the GEMM epilogue. */
typedef enum zq_act {
    ZQ_ACT_NONE = 0,
    ZQ_ACT_GELU = 1
} zq_act;

/* Which GEMM kernel zq_w8a8_gemm_dequant_ex runs. */
typedef enum zq_gemm_path {
    ZQ_PATH_AUTO = 0,       /* skinny kernel for M <= 32, tiled MFMA kernel otherwise */
    ZQ_PATH_TILED = 1,      /* LDS-tiled MFMA kernel (prefill shapes), any M */
    ZQ_PATH_SKINNY = 2      /* weight-streaming kernel (decode shapes), M <= 32 only */
} zq_gemm_path;

/* Largest K accepted: with codes in [-127, 127], |acc| <= 16129 K < 2^31. */
#define ZQ_MAX_K 131072

/*
 * zq_quantize_weights_grouped -- offline group-wise weight quantization.
 * [ZQN] group-wise weight quantization; [T36] 1.2.2 "用于权重矩阵的分组量化";
 * [SQ] 3.2 (weights are scaled by s, then quantized, offline).
 *
 *   W         [N x K], w_dtype ZQ_F32 or ZQ_F16, 16-byte aligned.
 *   smooth    [K] fp32 or NULL.  If given, the quantized matrix is
 *             W'[n, j] = fl32(W[n, j] * smooth[j]) (the weight side of the
 *             SmoothQuant fold); otherwise W' = W.
 *   group_rows G: group g is rows [g G, (g+1) G) by all K columns.
 *   Wq        [N x K] int8 out, 16-byte aligned.
 *   w_scales  [N / G] fp32 out: s_w[g] = fl32(max |W'| over the group / 127).
 *             The call also uses this array as its reduction scratch.
 * Requires N >= 1, 1 <= K <= ZQ_MAX_K, K % 16 == 0, G >= 1, N % G == 0.
 * W' must be finite.
 */
zq_status zq_quantize_weights_grouped(const void *W, zq_dtype w_dtype, const float *smooth,
                                      int64_t N, int64_t K, int64_t group_rows,
                                      int8_t *Wq, float *w_scales, hipStream_t stream);

/*
 * zq_ln_quant_per_token -- the fused prologue: LayerNorm or GeLU (or nothing)
 * in fp32 registers, then dynamic per-token absmax quantization.
 * [ZQN] kernel fusion "LN/GeLU + Quantize"; [T36] 1.2.2 token-wise
 * quantization with run-time ranges, fused with the preceding LayerNorm.
 *
 *   X         [M x K], x_dtype ZQ_F16 or ZQ_F32, 16-byte aligned.
 *   pre       ZQ_PRE_NONE / ZQ_PRE_LAYERNORM / ZQ_PRE_GELU.
 *   gamma, beta [K] fp32, used only for ZQ_PRE_LAYERNORM; NULL means 1 / 0.
 *   eps       LayerNorm epsilon (e.g. 1e-5).
 *   Xq        [M x K] int8 out, 16-byte aligned.
 *   x_scales  [M] fp32 out: s_x[m] = fl32(max_k |y[m, k]| / 127).
 * Requires M >= 1, 1 <= K <= ZQ_MAX_K, K % 16 == 0.  X must be finite: the
 * codes and scale of a token whose row holds an Inf or NaN are unspecified.
 */
zq_status zq_ln_quant_per_token(const void *X, zq_dtype x_dtype, int64_t M, int64_t K,
                                zq_pre pre, const float *gamma, const float *beta, float eps,
                                int8_t *Xq, float *x_scales, hipStream_t stream);

/*
 * zq_w8a8_gemm_dequant -- int8 x int8 -> int32 GEMM with the dequantization
 * fused into its epilogue.
 * [T36] 1.2.2: the INT32 accumulation is scaled by the activation and weight
 * scales before the FP16 write; [T36] 1.1.2 vector-wise: that scaling is the
 * outer product of the per-row and per-column scales; [IQ] MAC unit: the
 * bias joins the accumulation; [ZQN] kernel fusion "GeMM + DeQuantize".
 *
 *   acc[m, n] = sum_k Xq[m, k] Wq[n, k]                      (exact int32)
 *   v = s_x[m] * s_w[n / G] * acc[m, n] + bias[n]            (fp32)
 *   v = gelu(v) if act == ZQ_ACT_GELU
 *   Y[m, n] = fp16(v), round to nearest even                  (y_dtype ZQ_F16)
 *
 *   Xq [M x K], Wq [N x K] int8, 16-byte aligned; x_scales [M]; w_scales [N / G];
 *   bias [N] fp32 or NULL; Y [M x N], 16-byte aligned.
 *   y_dtype ZQ_F16 is the product path.  ZQ_I32 is a test mode: Y receives
 *   the raw int32 accumulators and x_scales, w_scales, bias and act are
 *   ignored (they may be NULL).
 * Requires M, N >= 1, 1 <= K <= ZQ_MAX_K, K % 16 == 0, G >= 1, N % G == 0,
 * N % 4 == 0 (outputs leave in whole 8-byte fp16 / 16-byte int32 pieces of
 * four columns; with G a multiple of 4, as every group size the pages give
 * is, N % G == 0 implies it).  Every call that runs this GEMM shares the rule.
 */
zq_status zq_w8a8_gemm_dequant(const int8_t *Xq, const float *x_scales, const int8_t *Wq,
                               const float *w_scales, int64_t group_rows, const float *bias,
                               zq_act act, int64_t M, int64_t N, int64_t K,
                               void *Y, zq_dtype y_dtype, hipStream_t stream);

/* As zq_w8a8_gemm_dequant, with the kernel chosen explicitly (tests, tuning).
 * ZQ_PATH_SKINNY with M > 32 returns ZQ_ERR_SHAPE. */
zq_status zq_w8a8_gemm_dequant_ex(const int8_t *Xq, const float *x_scales, const int8_t *Wq,
                                  const float *w_scales, int64_t group_rows, const float *bias,
                                  zq_act act, int64_t M, int64_t N, int64_t K,
                                  void *Y, zq_dtype y_dtype, zq_gemm_path path,
                                  hipStream_t stream);

/*
 * zq_linear_w8a8 -- the whole layer: prologue then GEMM + dequant, both on
 * `stream` with no host synchronisation in between ([ZQN] flowchart after
 * fusion).  The int8 codes and per-token scales pass through `workspace`.
 *
 *   Arguments as in the two calls above; Y is fp16 [M x N].
 *   workspace  device memory of at least zq_linear_workspace_bytes(M, K)
 *              bytes, 256-byte aligned, owned by the caller, overwritten.
 * Dispatches to the skinny (weight-streaming) GEMM when M <= 32.
 */
zq_status zq_linear_w8a8(const void *X, zq_dtype x_dtype, zq_pre pre, const float *gamma,
                         const float *beta, float eps, const int8_t *Wq, const float *w_scales,
                         int64_t group_rows, const float *bias, zq_act act,
                         int64_t M, int64_t N, int64_t K,
                         void *workspace, size_t workspace_bytes, void *Y, hipStream_t stream);

/*
 * zq_linear_w8a8_noalloc -- zq_linear_w8a8 for callers that cannot allocate
 * device memory or pass a workspace (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  The codes and scales go
 * to a fixed array inside the library instead of a caller workspace; the
 * call itself allocates nothing.
 *
 *   Arguments and results as zq_linear_w8a8, without workspace arguments.
 *   The array holds ZQ_NOALLOC_SCRATCH_BYTES (32 MiB) on each GPU the call
 *   runs on, from that GPU's first such call until the process ends.
 *   Requires zq_linear_workspace_bytes(M, K) <= ZQ_NOALLOC_SCRATCH_BYTES
 *   (e.g. 4096 tokens x 5120 features), else ZQ_ERR_WORKSPACE; other rules
 *   and errors as zq_linear_w8a8.  The device is the calling thread's current
 *   HIP device.
 *   Every call on one GPU shares that GPU's array: calls that may overlap on
 *   one GPU (other streams, other threads) race and give wrong results; calls
 *   in order on one stream are safe.  Not reentrant across streams.
 */
#define ZQ_NOALLOC_SCRATCH_BYTES (32u << 20)

zq_status zq_linear_w8a8_noalloc(const void *X, zq_dtype x_dtype, zq_pre pre, const float *gamma,
                                 const float *beta, float eps, const int8_t *Wq,
                                 const float *w_scales, int64_t group_rows, const float *bias,
                                 zq_act act, int64_t M, int64_t N, int64_t K, void *Y,
                                 hipStream_t stream);

/* Bytes of workspace zq_linear_w8a8 needs: the int8 codes (M*K rounded up to
 * 256) then the per-token scales (4*M rounded up to 256).  Returns 0 for
 * sizes that zq_linear_w8a8 would reject.  Layout: codes at offset 0, scales
 * right after the codes. */
size_t zq_linear_workspace_bytes(int64_t M, int64_t K);

/*
 * Packed weights for the weight-streaming (decode) GEMM.
 *
 * At decode shapes (M <= 32) the layer streams all of Wq from HBM once per
 * call and is bound by HBM bandwidth ("Integer Quantization: Deep Dive":
 * decoding is memory-bandwidth bound).  Read row-major, each workgroup's
 * slice of Wq is 32 rows one K apart; the packed layout stores what one
 * workgroup reads per pipeline step as one contiguous 16 KB run instead.
 * Packing is an offline re-layout of the quantized weights, like the
 * quantization itself ([T36] 1.2.2: weights are quantized ahead of time);
 * the codes and w_scales are unchanged, and results equal the row-major
 * calls bit for bit.
 *
 * Layout: with KS = ceil(K / 512), byte c of row r of block (b, s) is
 *   Wp[((b * KS + s) * 32 + r) * 512 + c] = Wq[(32 b + r) * K + 512 s + c],
 * or 0 where 32 b + r >= N or 512 s + c >= K.  b = 0 .. ceil(N / 32) - 1.
 */

/* Bytes of the packed layout: ceil(N / 32) * 32 * ceil(K / 512) * 512.
 * Returns 0 for sizes zq_pack_weights would reject. */
size_t zq_packed_weights_bytes(int64_t N, int64_t K);

/* zq_pack_weights -- offline: Wq [N x K] int8 -> Wp, zq_packed_weights_bytes(N, K)
 * bytes, both 16-byte aligned, not overlapping.  Requires N >= 1,
 * 1 <= K <= ZQ_MAX_K, K % 16 == 0. */
zq_status zq_pack_weights(const int8_t *Wq, int64_t N, int64_t K, int8_t *Wp,
                          hipStream_t stream);

/* As zq_w8a8_gemm_dequant (same arguments, y_dtype ZQ_F16 or the ZQ_I32 test
 * mode) with the weights given packed.  Runs the weight-streaming kernel:
 * requires M <= 32 (else ZQ_ERR_SHAPE). */
zq_status zq_w8a8_gemm_dequant_packed(const int8_t *Xq, const float *x_scales, const int8_t *Wp,
                                      const float *w_scales, int64_t group_rows,
                                      const float *bias, zq_act act, int64_t M, int64_t N,
                                      int64_t K, void *Y, zq_dtype y_dtype, hipStream_t stream);

/* As zq_linear_w8a8 with the weights given packed; requires M <= 32. */
zq_status zq_linear_w8a8_packed(const void *X, zq_dtype x_dtype, zq_pre pre,
                                const float *gamma, const float *beta, float eps,
                                const int8_t *Wp, const float *w_scales, int64_t group_rows,
                                const float *bias, zq_act act, int64_t M, int64_t N, int64_t K,
                                void *workspace, size_t workspace_bytes, void *Y,
                                hipStream_t stream);

/*
 * zq_linear_w8a8_unfused -- the same layer in the unfused order, for measuring
 * what the fusion saves (ZeroQuant reading notes, kernel-fusion figure, the
 * flow before fusion): (1) LN/GeLU writes y as an fp16 tensor, (2) a separate
 * kernel quantizes that tensor per token, (3) the int8 GEMM writes its int32
 * accumulators, (4) a separate kernel dequantizes them (+ bias, + GeLU) to
 * fp16.  Not the product path: zq_linear_w8a8 computes the fused form.
 * Results differ from zq_linear_w8a8 only by the fp16 rounding of y between
 * (1) and (2); steps (3)-(4) give the fused epilogue's bits for the same codes.
 *
 *   Arguments as zq_linear_w8a8.  workspace: zq_linear_unfused_workspace_bytes
 *   (M, N, K) bytes, 256-byte aligned, overwritten; layout y fp16 [M x K],
 *   codes int8 [M x K], scales fp32 [M], accumulators int32 [M x N], each at
 *   the next 256-byte boundary.
 */
zq_status zq_linear_w8a8_unfused(const void *X, zq_dtype x_dtype, zq_pre pre,
                                 const float *gamma, const float *beta, float eps,
                                 const int8_t *Wq, const float *w_scales, int64_t group_rows,
                                 const float *bias, zq_act act, int64_t M, int64_t N, int64_t K,
                                 void *workspace, size_t workspace_bytes, void *Y,
                                 hipStream_t stream);

/* Bytes of workspace zq_linear_w8a8_unfused needs (see above); 0 for sizes it
 * would reject. */
size_t zq_linear_unfused_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * zq_ffn_w8a8 -- a transformer FFN block, chained on one stream:
 *   H = GeLU(s_x1 s_w1 (quant(LN(X)) W1q^T) + b1)       [M x F] fp16   (FFN-up)
 *   Y =      s_x2 s_w2 (quant(H)     W2q^T) + b2        [M x K] fp16   (FFN-down)
 * i.e. zq_linear_w8a8 with LayerNorm and the GeLU epilogue, then
 * zq_linear_w8a8 without a pre-op on H ([ZQN] flowchart: LN+Quantize,
 * GeMM+DeQuantize, GeLU, Quantize, GeMM+DeQuantize; [T36] 1.2.2).  The
 * FFN-up GEMM's epilogue also writes, for every token, max |H[m, :]| over each
 * of its column groups (plain stores of partial maxima, no atomics), so H's
 * quantizer combines a few partials per token instead of reducing H; the
 * result equals the two zq_linear_w8a8 calls bit for bit.
 *
 *   X [M x K] (ZQ_F16 / ZQ_F32); gamma, beta [K] or NULL; W1q [F x K] int8 with
 *   w1_scales [F / group_rows1] and bias1 [F] or NULL; W2q [K x F] int8 with
 *   w2_scales [K / group_rows2] and bias2 [K] or NULL; Y [M x K] fp16.
 *   workspace  zq_ffn_workspace_bytes(M, K, F) bytes, 256-byte aligned,
 *              overwritten (H, the partial maxima, codes and scales of both layers).
 * Requires each layer to meet zq_linear_w8a8's rules.
 */
zq_status zq_ffn_w8a8(const void *X, zq_dtype x_dtype, const float *gamma, const float *beta,
                      float eps, const int8_t *W1q, const float *w1_scales, int64_t group_rows1,
                      const float *bias1, const int8_t *W2q, const float *w2_scales,
                      int64_t group_rows2, const float *bias2, int64_t M, int64_t K, int64_t F,
                      void *workspace, size_t workspace_bytes, void *Y, hipStream_t stream);

/* Bytes of workspace zq_ffn_w8a8 needs; 0 for sizes it would reject. */
size_t zq_ffn_workspace_bytes(int64_t M, int64_t K, int64_t F);

/*
 * FP8 variant ("探秘Transformer系列之（36）--- 大模型量化方案", the ZeroQuant-FP
 * paragraph: FP8 activations; every scale factor a power of two, kept within
 * one compute group).  Codes are OCP 8-bit E4M3 ("FN": bias 7, no
 * infinities, largest finite 448) stored one per byte; scales are powers of
 * two: for a vector with absmax a > 0 the scale is the smallest 2^e with
 * a <= 448 * 2^e (nothing clips), and a code is the E4M3 value nearest to
 * v / 2^e (an exact scaling), ties to even; a = 0 gives scale 0 and codes 0.
 * Activations: one scale per token, after the fused LN/GeLU (as the int8
 * prologue).  Weights: one scale per group of G output rows (as the int8
 * weights).  The GEMM multiplies the codes on the FP8 matrix cores with fp32
 * accumulation (not exact, unlike the int8 path), then the same epilogue:
 * Y = fp16(s_x[m] s_w[n / G] acc + bias[n]), optional GeLU.  Shapes,
 * alignment and workspace rules are those of the int8 calls.
 */
zq_status zq_quantize_weights_grouped_fp8(const void *W, zq_dtype w_dtype, const float *smooth,
                                          int64_t N, int64_t K, int64_t group_rows,
                                          uint8_t *Wq8, float *w_scales, hipStream_t stream);

zq_status zq_ln_quant_per_token_fp8(const void *X, zq_dtype x_dtype, int64_t M, int64_t K,
                                    zq_pre pre, const float *gamma, const float *beta, float eps,
                                    uint8_t *Xq8, float *x_scales, hipStream_t stream);

/* y_dtype ZQ_F16 (the product) or ZQ_F32: Y receives the raw fp32
 * accumulators (test mode; scales, bias and act ignored). */
zq_status zq_fp8_gemm_dequant(const uint8_t *Xq8, const float *x_scales, const uint8_t *Wq8,
                              const float *w_scales, int64_t group_rows, const float *bias,
                              zq_act act, int64_t M, int64_t N, int64_t K, void *Y,
                              zq_dtype y_dtype, hipStream_t stream);

/* The FP8 layer; workspace as zq_linear_workspace_bytes(M, K). */
zq_status zq_linear_w8a8_fp8(const void *X, zq_dtype x_dtype, zq_pre pre, const float *gamma,
                             const float *beta, float eps, const uint8_t *Wq8,
                             const float *w_scales, int64_t group_rows, const float *bias,
                             zq_act act, int64_t M, int64_t N, int64_t K, void *workspace,
                             size_t workspace_bytes, void *Y, hipStream_t stream);

/* As zq_linear_w8a8_fp8 with the codes packed by zq_pack_weights; M <= 32. */
zq_status zq_linear_w8a8_fp8_packed(const void *X, zq_dtype x_dtype, zq_pre pre,
                                    const float *gamma, const float *beta, float eps,
                                    const uint8_t *Wp8, const float *w_scales,
                                    int64_t group_rows, const float *bias, zq_act act, int64_t M,
                                    int64_t N, int64_t K, void *workspace,
                                    size_t workspace_bytes, void *Y, hipStream_t stream);

/*
 * Mixed-precision decomposition ("探秘Transformer系列之（36）--- 大模型量化方案"
 * 1.1 LLM.int8(), "方案" and "混合精度分解"): the alternative to the SmoothQuant
 * fold for activations with outlier feature dimensions.
 *
 *   y = LN / GeLU / x as in zq_ln_quant_per_token (fp32).
 *   O = { j : |y[m, j]| > alpha for some token m of the batch }, ascending
 *       (strict; alpha = 6.0 is the page's setting; a NaN alpha selects no
 *       column, a negative one every column).
 *   INT8 part: per token, s_x[m] = fl32(max_{j not in O} |y[m, j]| / 127) and
 *       codes as usual on the columns outside O, code 0 on the columns in O;
 *       the weights are the layer's group-wise int8 codes (group_rows = 1 is
 *       the page's per-output-channel scale), quantized over all K offline.
 *   FP16 part: sum_{j in O} fp16(y[m, j]) * fp16(W[n, j]), from the fp16
 *       weights W16t (zq_pack_outlier_weights).
 *   Y[m, n] = fp16(act(s_x[m] s_w[n / G] acc[m, n] + fp16 part + bias[n])),
 *       the sum and the GeLU in fp32.
 *
 * Device layouts:
 *   slot  int32 [K], 16-byte aligned: position of column j in O, or -1.
 *   cols  int32 [K + 1]: cols[0] = |O|, cols[1 .. |O|] the columns of O.
 *   XO    fp16 [M x K], 16-byte aligned: token m's value of the p-th column
 *         of O at XO[m * K + p], p < |O| (the rest of each row is not used;
 *         the row length K is the bound on |O|).
 *   W16t  fp16 [K x N], 16-byte aligned: W transposed (input-channel major),
 *         so each outlier column is one contiguous run of N values.
 * Shapes, alignment and error rules are those of the int8 calls; Y is fp16.
 */

/* Offline: W [N x K] (ZQ_F32 / ZQ_F16) -> W16t [K x N] fp16, nearest-even. */
zq_status zq_pack_outlier_weights(const void *W, zq_dtype w_dtype, int64_t N, int64_t K,
                                  void *W16t, hipStream_t stream);

/* The outlier set of a batch: writes slot and cols (slot is also the scratch
 * of the search). */
zq_status zq_outlier_columns(const void *X, zq_dtype x_dtype, int64_t M, int64_t K, zq_pre pre,
                             const float *gamma, const float *beta, float eps, float alpha,
                             int32_t *slot, int32_t *cols, hipStream_t stream);

/* The prologue of the INT8 part (codes, scales) plus the outlier values XO,
 * given slot from zq_outlier_columns for the same batch. */
zq_status zq_ln_quant_decomp(const void *X, zq_dtype x_dtype, int64_t M, int64_t K, zq_pre pre,
                             const float *gamma, const float *beta, float eps,
                             const int32_t *slot, int8_t *Xq, float *x_scales, void *XO,
                             hipStream_t stream);

/* INT8 GEMM with the dequantization and the FP16 outlier product in its
 * epilogue (fp16 Y). */
zq_status zq_w8a8_gemm_decomp(const int8_t *Xq, const float *x_scales, const int8_t *Wq,
                              const float *w_scales, int64_t group_rows, const int32_t *cols,
                              const void *XO, const void *W16t, const float *bias, zq_act act,
                              int64_t M, int64_t N, int64_t K, void *Y, hipStream_t stream);

/* The whole decomposed layer: outlier search, prologue, GEMM.  workspace is
 * 256-byte aligned, at least zq_linear_decomp_workspace_bytes(M, K) bytes. */
zq_status zq_linear_w8a8_decomp(const void *X, zq_dtype x_dtype, zq_pre pre, const float *gamma,
                                const float *beta, float eps, float alpha, const int8_t *Wq,
                                const float *w_scales, int64_t group_rows, const void *W16t,
                                const float *bias, zq_act act, int64_t M, int64_t N, int64_t K,
                                void *workspace, size_t workspace_bytes, void *Y,
                                hipStream_t stream);

/* slot [K] | cols [K + 1] | codes [M K] | scales [M] | XO fp16 [M K], each
 * part rounded up to 256 bytes; 0 for invalid sizes. */
size_t zq_linear_decomp_workspace_bytes(int64_t M, int64_t K);

/*
 * zq_smoothquant_factors -- offline SmoothQuant calibration and LayerNorm fold.
 * [SQ] 2.2: Y = (X diag(s)^-1)(diag(s) W), s per input channel; [SQ] 3.2:
 * the factors are computed offline from activation statistics.
 *
 *   Statistics: a_j = max_m |LN(X)[m, j]| with gamma = 1, beta = 0 (the
 *   linear's actual input), w_j = max_n |W[n, j]|;
 *   smooth[j] = fl32(sqrt(a_j / w_j)), or 1 when a_j or w_j is 0.
 *   Fold: gamma_out[j] = fl32(gamma[j] / smooth[j]), beta_out[j] = fl32(beta[j] / smooth[j])
 *   (gamma / beta NULL mean 1 / 0), so that LN with gamma_out, beta_out equals
 *   LN(X) diag(smooth)^-1.  The weight side is applied by passing `smooth`
 *   to zq_quantize_weights_grouped.
 *
 *   X [M x K] (ZQ_F16 / ZQ_F32), W [N x K] (ZQ_F32 / ZQ_F16), both 16-byte aligned.
 *   smooth, gamma_out, beta_out [K] fp32 out.
 *   workspace  at least zq_smoothquant_workspace_bytes(M, K) bytes, 256-byte aligned.
 * Requires M, N >= 1, 1 <= K <= ZQ_MAX_K, K % 16 == 0; X and W finite.
 */
zq_status zq_smoothquant_factors(const void *X, zq_dtype x_dtype, int64_t M, int64_t K, float eps,
                                 const void *W, zq_dtype w_dtype, int64_t N,
                                 const float *gamma, const float *beta,
                                 float *smooth, float *gamma_out, float *beta_out,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace zq_smoothquant_factors needs (8*M + 8*K, rounded up to 256). */
size_t zq_smoothquant_workspace_bytes(int64_t M, int64_t K);

/* A static, human-readable name for a status code. */
const char *zq_status_str(zq_status status);

#ifdef __cplusplus
}
#endif

#endif /* ZQ_H */
