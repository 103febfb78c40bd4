// Internal launcher interface between the C ABI (zq_api.hip) and the gfx950
// kernels.  Not installed, not part of the ABI.  Every launcher assumes the
// arguments were validated by the caller and returns the HIP launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zq {

// The fp16 part of the mixed-precision decomposition, as the GEMM epilogues
// read it: cols[0] = P, cols[1 + p] = the p-th outlier column; xo [M x K]
// fp16 holds token m's value of column cols[1 + p] at xo[m * K + p]; wt
// [K x N] fp16 is W transposed (for a launch over a column range of Y, wt
// points at the range's first column and its rows keep Y's row stride).
struct OutlierOperands {
    const int32_t *cols;
    const _Float16 *xo;
    const _Float16 *wt;
};

// Prologue: LN / GeLU / none in fp32, then per-token absmax quantization
// (int8 codes, or with fp8 OCP E4M3 codes and power-of-two scales).
hipError_t launch_ln_quant(const void *X, bool x_f16, int64_t M, int64_t K, int pre,
                           const float *gamma, const float *beta, float eps,
                           int8_t *Xq, float *x_scales, hipStream_t stream, bool fp8 = false);

// Quantization of fp16 rows whose absmax is the maximum of partial maxima
// part[m * groups + j] (from a GEMM epilogue's row_part output).
hipError_t launch_quant_rows_part(const _Float16 *Y, int64_t M, int64_t K, const float *part,
                                  int64_t groups, int8_t *Xq, float *x_scales,
                                  hipStream_t stream);

// The op alone, its result stored as fp16 (the unfused order).
hipError_t launch_ln_to_f16(const void *X, bool x_f16, int64_t M, int64_t K, int pre,
                            const float *gamma, const float *beta, float eps, _Float16 *Y16,
                            hipStream_t stream);

// Dequantization of int32 accumulators as its own kernel (the unfused order).
hipError_t launch_dequant(const int32_t *acc, const float *x_scales, const float *w_scales,
                          int64_t G, const float *bias, int act, int64_t M, int64_t N, void *Y,
                          hipStream_t stream);

// Tiled MFMA GEMM (prefill shapes) with the fused dequant epilogue.
// out_i32 selects the raw-accumulator test mode.
// row_part (optional, fp16 output only): partial maxima of |Y[m, :]|,
// row_part[m * gemm_tiled_row_groups(M, N) + j] over column group j; every
// entry of a row m < M is written (plain stores, nothing to clear first).
hipError_t launch_gemm_tiled(const int8_t *Xq, const float *x_scales, const int8_t *Wq,
                             const float *w_scales, int64_t G, const float *bias, int act,
                             int64_t M, int64_t N, int64_t K, void *Y, bool out_i32,
                             hipStream_t stream, float *row_part = nullptr);
int64_t gemm_tiled_row_groups(int64_t M, int64_t N);

// The FP8 variant of the tiled GEMM: OCP E4M3 operands, fp32 accumulation,
// same epilogue; out_raw writes the fp32 accumulators.
hipError_t launch_gemm_tiled_fp8(const int8_t *Xq, const float *x_scales, const int8_t *Wq,
                                 const float *w_scales, int64_t G, const float *bias, int act,
                                 int64_t M, int64_t N, int64_t K, void *Y, bool out_raw,
                                 hipStream_t stream);

// Weight-streaming MFMA GEMM for M <= 32 (decode shapes), same epilogue;
// row_part as for the tiled GEMM, with gemm_skinny_row_groups(N) groups.
hipError_t launch_gemm_skinny(const int8_t *Xq, const float *x_scales, const int8_t *Wq,
                              const float *w_scales, int64_t G, const float *bias, int act,
                              int64_t M, int64_t N, int64_t K, void *Y, bool out_i32,
                              hipStream_t stream, float *row_part = nullptr);
int64_t gemm_skinny_row_groups(int64_t N);

// The same kernel reading weights in the packed layout of launch_pack_weights.
hipError_t launch_gemm_skinny_packed(const int8_t *Xq, const float *x_scales, const int8_t *Wp,
                                     const float *w_scales, int64_t G, const float *bias, int act,
                                     int64_t M, int64_t N, int64_t K, void *Y, bool out_i32,
                                     hipStream_t stream);

// The FP8 variant of the weight-streaming GEMM (row-major or packed weights).
hipError_t launch_gemm_skinny_fp8(const int8_t *Xq, const float *x_scales, const int8_t *Wq,
                                  const float *w_scales, int64_t G, const float *bias, int act,
                                  int64_t M, int64_t N, int64_t K, void *Y, bool out_raw,
                                  bool packed, hipStream_t stream);

// Mixed-precision decomposition (outlier columns in fp16).
// Outlier set: slot [K] and cols [K + 1] as k_outlier_compact leaves them
// (cols[0] = |O|, cols[1..] ascending; slot[j] = position or -1).
hipError_t launch_outlier_columns(const void *X, bool x_f16, int64_t M, int64_t K, int pre,
                                  const float *gamma, const float *beta, float eps, float alpha,
                                  int32_t *slot, int32_t *cols, hipStream_t stream);
// The marking pass alone.  slot must be cleared first unless
// outlier_detect_writes_all(M, K, pre), in which case the pass writes every
// entry (1 or 0) itself.
bool outlier_detect_writes_all(int64_t M, int64_t K, int pre);
hipError_t launch_outlier_detect(const void *X, bool x_f16, int64_t M, int64_t K, int pre,
                                 const float *gamma, const float *beta, float eps, float alpha,
                                 int32_t *slot, hipStream_t stream);
// Prologue over the non-outlier columns; outlier values to XO [M x K] fp16 at
// XO[m * K + position].
hipError_t launch_ln_quant_decomp(const void *X, bool x_f16, int64_t M, int64_t K, int pre,
                                  const float *gamma, const float *beta, float eps,
                                  const int32_t *slot, int8_t *Xq, float *x_scales, _Float16 *XO,
                                  hipStream_t stream);
// Weight-streaming GEMM (M <= 32, row-major weights) whose epilogue adds the
// fp16 outlier product (fp16 output).
hipError_t launch_gemm_skinny_decomp(const int8_t *Xq, const float *x_scales, const int8_t *Wq,
                                     const float *w_scales, int64_t G, const float *bias, int act,
                                     int64_t M, int64_t N, int64_t K, const int32_t *cols,
                                     const _Float16 *XO, const _Float16 *W16t, void *Y,
                                     hipStream_t stream);
// Tiled GEMM whose epilogue adds the fp16 outlier product (fp16 output).
hipError_t launch_gemm_tiled_decomp(const int8_t *Xq, const float *x_scales, const int8_t *Wq,
                                    const float *w_scales, int64_t G, const float *bias, int act,
                                    int64_t M, int64_t N, int64_t K, const int32_t *cols,
                                    const _Float16 *XO, const _Float16 *W16t, void *Y,
                                    hipStream_t stream);
// Offline: W [N x K] (fp32 / fp16) -> W16t [K x N] fp16.
hipError_t launch_pack_outlier_weights(const void *W, bool w_f16, int64_t N, int64_t K,
                                       _Float16 *W16t, hipStream_t stream);

// Offline re-layout of Wq [N x K] into 32-row x 512-byte blocks (zero padded)
// that the weight-streaming kernel reads as contiguous 16 KB runs.
int64_t packed_weights_bytes(int64_t N, int64_t K);
hipError_t launch_pack_weights(const int8_t *Wq, int64_t N, int64_t K, int8_t *Wp,
                               hipStream_t stream);

// Offline group-wise weight quantization (optionally W * diag(smooth)).
// With fp8: OCP E4M3 codes and power-of-two group scales.
hipError_t launch_quantize_weights(const void *W, bool w_f16, const float *smooth,
                                   int64_t N, int64_t K, int64_t G, int8_t *Wq,
                                   float *w_scales, hipStream_t stream, bool fp8 = false);

// Offline SmoothQuant factors and LayerNorm fold.  ws holds 2*M floats of
// per-token statistics followed by 2*K uint32 channel maxima.
hipError_t launch_smooth_factors(const void *X, bool x_f16, int64_t M, int64_t K, float eps,
                                 const void *W, bool w_f16, int64_t N,
                                 const float *gamma, const float *beta, float *smooth,
                                 float *gamma_out, float *beta_out, void *ws,
                                 hipStream_t stream);

}  // namespace zq
