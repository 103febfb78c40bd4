// C ABI of libzq (declared in include/zq.h): host-side validation, dispatch
// to the gfx950 kernels, and HIP error mapping.  Every argument is checked
// before anything is enqueued; on error nothing is enqueued.
#include "zq.h"
#include "zq_kernels.h"

#include <mutex>

#define ZQ_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int64_t kSkinnyMaxM = 32;

bool aligned16(const void *p)
{
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

bool aligned16_or_null(const void *p)
{
    return p == nullptr || aligned16(p);
}

size_t round_up(size_t v, size_t a)
{
    return (v + a - 1) / a * a;
}

zq_status map_hip(hipError_t e)
{
    return e == hipSuccess ? ZQ_OK : ZQ_ERR_HIP;
}

// An error left pending on this thread by earlier HIP work belongs to the
// caller: the call then returns ZQ_ERR_HIP before enqueueing anything and
// leaves that error pending (peek, not get), so the caller still reads it,
// and a launch failure this library reports is always its own.
bool hip_error_pending()
{
    return hipPeekAtLastError() != hipSuccess;
}

bool k_ok(int64_t K)
{
    return K >= 1 && K <= ZQ_MAX_K && K % 16 == 0;
}

zq_status check_gemm(const int8_t *Xq, const float *x_scales, const int8_t *Wq,
                     const float *w_scales, int64_t G, zq_act act, int64_t M, int64_t N,
                     int64_t K, const void *Y, zq_dtype y_dtype, const float *bias)
{
    if (!Xq || !Wq || !Y)
        return ZQ_ERR_NULL;
    if (y_dtype != ZQ_F16 && y_dtype != ZQ_I32)
        return ZQ_ERR_DTYPE;
    if (act != ZQ_ACT_NONE && act != ZQ_ACT_GELU)
        return ZQ_ERR_DTYPE;
    if (y_dtype == ZQ_F16 && (!x_scales || !w_scales))
        return ZQ_ERR_NULL;
    if (M < 1 || N < 1 || !k_ok(K) || G < 1 || N % G != 0 || N % 4 != 0)
        return ZQ_ERR_SHAPE;
    if (M > INT32_MAX || N > INT32_MAX || M * K > (int64_t)1 << 40 || N * K > (int64_t)1 << 40 ||
        M * N > (int64_t)1 << 40)
        return ZQ_ERR_SHAPE;
    if (!aligned16(Xq) || !aligned16(Wq) || !aligned16(Y))
        return ZQ_ERR_ALIGN;
    (void)bias;
    return ZQ_OK;
}

zq_status check_prologue(const void *X, zq_dtype x_dtype, int64_t M, int64_t K, zq_pre pre,
                         const float *gamma, const float *beta, const int8_t *Xq,
                         const float *x_scales)
{
    if (!X || !Xq || !x_scales)
        return ZQ_ERR_NULL;
    if (x_dtype != ZQ_F16 && x_dtype != ZQ_F32)
        return ZQ_ERR_DTYPE;
    if (pre != ZQ_PRE_NONE && pre != ZQ_PRE_LAYERNORM && pre != ZQ_PRE_GELU)
        return ZQ_ERR_DTYPE;
    if (M < 1 || !k_ok(K) || M > INT32_MAX || M * K > (int64_t)1 << 40)
        return ZQ_ERR_SHAPE;
    if (!aligned16(X) || !aligned16(Xq))
        return ZQ_ERR_ALIGN;
    if (pre == ZQ_PRE_LAYERNORM && (!aligned16_or_null(gamma) || !aligned16_or_null(beta)))
        return ZQ_ERR_ALIGN;
    return ZQ_OK;
}

zq_status gemm_dispatch(const int8_t *Xq, const float *x_scales, const int8_t *Wq,
                        const float *w_scales, int64_t G, const float *bias, zq_act act,
                        int64_t M, int64_t N, int64_t K, void *Y, zq_dtype y_dtype,
                        zq_gemm_path path, hipStream_t stream)
{
    const bool i32 = y_dtype == ZQ_I32;
    const bool skinny = path == ZQ_PATH_SKINNY || (path == ZQ_PATH_AUTO && M <= kSkinnyMaxM);
    hipError_t e;
    if (skinny)
        e = zq::launch_gemm_skinny(Xq, x_scales, Wq, w_scales, G, bias, (int)act, M, N, K, Y, i32,
                                   stream);
    else
        e = zq::launch_gemm_tiled(Xq, x_scales, Wq, w_scales, G, bias, (int)act, M, N, K, Y, i32,
                                  stream);
    return map_hip(e);
}

}  // namespace

ZQ_API const char *zq_status_str(zq_status s)
{
    switch (s) {
    case ZQ_OK: return "ZQ_OK";
    case ZQ_ERR_NULL: return "ZQ_ERR_NULL: a required pointer is NULL";
    case ZQ_ERR_SHAPE: return "ZQ_ERR_SHAPE: a size is out of range or not a required multiple";
    case ZQ_ERR_ALIGN: return "ZQ_ERR_ALIGN: a pointer is not 16-byte aligned";
    case ZQ_ERR_DTYPE: return "ZQ_ERR_DTYPE: unsupported dtype or op";
    case ZQ_ERR_WORKSPACE: return "ZQ_ERR_WORKSPACE: workspace missing or too small";
    case ZQ_ERR_HIP: return "ZQ_ERR_HIP: the HIP runtime reported an error";
    case ZQ_ERR_UNSUPPORTED: return "ZQ_ERR_UNSUPPORTED: not implemented";
    }
    return "unknown zq_status";
}

ZQ_API zq_status zq_quantize_weights_grouped(const void *W, zq_dtype w_dtype, const float *smooth,
                                             int64_t N, int64_t K, int64_t group_rows, int8_t *Wq,
                                             float *w_scales, hipStream_t stream)
{
    if (!W || !Wq || !w_scales)
        return ZQ_ERR_NULL;
    if (w_dtype != ZQ_F32 && w_dtype != ZQ_F16)
        return ZQ_ERR_DTYPE;
    if (N < 1 || !k_ok(K) || group_rows < 1 || N % group_rows != 0 || N > INT32_MAX ||
        N * K > (int64_t)1 << 40)
        return ZQ_ERR_SHAPE;
    if (!aligned16(W) || !aligned16(Wq))
        return ZQ_ERR_ALIGN;
    if (hip_error_pending())
        return ZQ_ERR_HIP;
    return map_hip(zq::launch_quantize_weights(W, w_dtype == ZQ_F16, smooth, N, K, group_rows, Wq,
                                               w_scales, stream));
}

ZQ_API zq_status zq_ln_quant_per_token(const void *X, zq_dtype x_dtype, int64_t M, int64_t K,
                                       zq_pre pre, const float *gamma, const float *beta,
                                       float eps, int8_t *Xq, float *x_scales, hipStream_t stream)
{
    zq_status st = check_prologue(X, x_dtype, M, K, pre, gamma, beta, Xq, x_scales);
    if (st != ZQ_OK)
        return st;
    if (hip_error_pending())
        return ZQ_ERR_HIP;
    return map_hip(zq::launch_ln_quant(X, x_dtype == ZQ_F16, M, K, (int)pre,
                                       pre == ZQ_PRE_LAYERNORM ? gamma : nullptr,
                                       pre == ZQ_PRE_LAYERNORM ? beta : nullptr, eps, Xq,
                                       x_scales, stream));
}

ZQ_API zq_status zq_w8a8_gemm_dequant_ex(const int8_t *Xq, const float *x_scales,
                                         const int8_t *Wq, const float *w_scales,
                                         int64_t group_rows, const float *bias, zq_act act,
                                         int64_t M, int64_t N, int64_t K, void *Y,
                                         zq_dtype y_dtype, zq_gemm_path path, hipStream_t stream)
{
    zq_status st = check_gemm(Xq, x_scales, Wq, w_scales, group_rows, act, M, N, K, Y, y_dtype,
                              bias);
    if (st != ZQ_OK)
        return st;
    if (path != ZQ_PATH_AUTO && path != ZQ_PATH_TILED && path != ZQ_PATH_SKINNY)
        return ZQ_ERR_DTYPE;
    if (path == ZQ_PATH_SKINNY && M > kSkinnyMaxM)
        return ZQ_ERR_SHAPE;
    if (hip_error_pending())
        return ZQ_ERR_HIP;
    return gemm_dispatch(Xq, x_scales, Wq, w_scales, group_rows, bias, act, M, N, K, Y, y_dtype,
                         path, stream);
}

ZQ_API zq_status zq_w8a8_gemm_dequant(const int8_t *Xq, const float *x_scales, const int8_t *Wq,
                                      const float *w_scales, int64_t group_rows,
                                      const float *bias, zq_act act, int64_t M, int64_t N,
                                      int64_t K, void *Y, zq_dtype y_dtype, hipStream_t stream)
{
    return zq_w8a8_gemm_dequant_ex(Xq, x_scales, Wq, w_scales, group_rows, bias, act, M, N, K, Y,
                                   y_dtype, ZQ_PATH_AUTO, stream);
}

// Workspace of zq_linear_w8a8: codes [M*K] | scales [M], each part starting on
// a 256-byte boundary.
ZQ_API size_t zq_linear_workspace_bytes(int64_t M, int64_t K)
{
    if (M < 1 || !k_ok(K) || M > INT32_MAX || M * K > (int64_t)1 << 40)
        return 0;
    return round_up((size_t)(M * K), 256) + round_up(4 * (size_t)M, 256);
}

namespace {

zq_status linear_impl(const void *X, zq_dtype x_dtype, zq_pre pre, const float *gamma,
                      const float *beta, float eps, const int8_t *Wq, const float *w_scales,
                      int64_t group_rows, const float *bias, zq_act act, int64_t M, int64_t N,
                      int64_t K, void *workspace, size_t workspace_bytes, void *Y, bool packed,
                      hipStream_t stream)
{
    if (!X || !Wq || !w_scales || !Y)
        return ZQ_ERR_NULL;
    if (!workspace)
        return ZQ_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return ZQ_ERR_ALIGN;
    const size_t need = zq_linear_workspace_bytes(M, K);
    const size_t codes_bytes = round_up((size_t)(M > 0 && K > 0 ? M * K : 0), 256);
    int8_t *Xq = static_cast<int8_t *>(workspace);
    float *x_scales = reinterpret_cast<float *>(static_cast<char *>(workspace) + codes_bytes);
    zq_status st = check_prologue(X, x_dtype, M, K, pre, gamma, beta, Xq, x_scales);
    if (st != ZQ_OK)
        return st;
    st = check_gemm(Xq, x_scales, Wq, w_scales, group_rows, act, M, N, K, Y, ZQ_F16, bias);
    if (st != ZQ_OK)
        return st;
    if (packed && M > kSkinnyMaxM)
        return ZQ_ERR_SHAPE;
    if (workspace_bytes < need)
        return ZQ_ERR_WORKSPACE;
    if (hip_error_pending())
        return ZQ_ERR_HIP;
    st = map_hip(zq::launch_ln_quant(X, x_dtype == ZQ_F16, M, K, (int)pre,
                                     pre == ZQ_PRE_LAYERNORM ? gamma : nullptr,
                                     pre == ZQ_PRE_LAYERNORM ? beta : nullptr, eps, Xq, x_scales,
                                     stream));
    if (st != ZQ_OK)
        return st;
    if (packed)
        return map_hip(zq::launch_gemm_skinny_packed(Xq, x_scales, Wq, w_scales, group_rows, bias,
                                                     (int)act, M, N, K, Y, false, stream));
    return gemm_dispatch(Xq, x_scales, Wq, w_scales, group_rows, bias, act, M, N, K, Y, ZQ_F16,
                         ZQ_PATH_AUTO, stream);
}

}  // namespace

ZQ_API zq_status zq_linear_w8a8(const void *X, zq_dtype x_dtype, zq_pre pre, const float *gamma,
                                const float *beta, float eps, const int8_t *Wq,
                                const float *w_scales, int64_t group_rows, const float *bias,
                                zq_act act, int64_t M, int64_t N, int64_t K, void *workspace,
                                size_t workspace_bytes, void *Y, hipStream_t stream)
{
    return linear_impl(X, x_dtype, pre, gamma, beta, eps, Wq, w_scales, group_rows, bias, act, M,
                       N, K, workspace, workspace_bytes, Y, false, stream);
}

ZQ_API zq_status zq_linear_w8a8_packed(const void *X, zq_dtype x_dtype, zq_pre pre,
                                       const float *gamma, const float *beta, float eps,
                                       const int8_t *Wp, const float *w_scales,
                                       int64_t group_rows, const float *bias, zq_act act,
                                       int64_t M, int64_t N, int64_t K, void *workspace,
                                       size_t workspace_bytes, void *Y, hipStream_t stream)
{
    return linear_impl(X, x_dtype, pre, gamma, beta, eps, Wp, w_scales, group_rows, bias, act, M,
                       N, K, workspace, workspace_bytes, Y, true, stream);
}

// ---- The layer for callers that cannot allocate ----
//
// zq_linear_w8a8_noalloc runs zq_linear_w8a8 with its workspace (the int8
// codes and the per-token scales) in a fixed device array of this file
// instead of a caller buffer.  Each GPU the library runs on holds its own copy
// of the array until the process ends.  In host code `scratch` names a
// host-side stand-in, never the device memory: the device address is looked
// up once per device with hipGetSymbolAddress and only that address is
// passed on.
static __device__ __align__(256) uint8_t scratch[ZQ_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// The device address of the scratch array on the current device.  The first
// call on a device, with that device current, looks it up; later calls reuse
// it.  Nothing is allocated here or anywhere on this path.
zq_status scratch_on_current_device(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();  // this call's own failure, reported as ZQ_ERR_HIP
        return ZQ_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices)
        return ZQ_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return ZQ_ERR_HIP;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return ZQ_OK;
}

}  // namespace

ZQ_API zq_status zq_linear_w8a8_noalloc(const void *X, zq_dtype x_dtype, zq_pre pre,
                                        const float *gamma, const float *beta, float eps,
                                        const int8_t *Wq, const float *w_scales,
                                        int64_t group_rows, const float *bias, zq_act act,
                                        int64_t M, int64_t N, int64_t K, void *Y,
                                        hipStream_t stream)
{
    if (!X || !Wq || !w_scales || !Y)
        return ZQ_ERR_NULL;
    const size_t need = zq_linear_workspace_bytes(M, K);
    if (need == 0)
        return ZQ_ERR_SHAPE;
    if (need > (size_t)ZQ_NOALLOC_SCRATCH_BYTES)
        return ZQ_ERR_WORKSPACE;
    if (hip_error_pending())
        return ZQ_ERR_HIP;
    void *ws = nullptr;
    const zq_status st = scratch_on_current_device(&ws);
    if (st != ZQ_OK)
        return st;
    // The prologue writes every code and scale the GEMM then reads, so nothing
    // in the array needs clearing between calls.
    return linear_impl(X, x_dtype, pre, gamma, beta, eps, Wq, w_scales, group_rows, bias, act, M,
                       N, K, ws, (size_t)ZQ_NOALLOC_SCRATCH_BYTES, Y, false, stream);
}

ZQ_API size_t zq_packed_weights_bytes(int64_t N, int64_t K)
{
    if (N < 1 || !k_ok(K) || N > INT32_MAX || N * K > (int64_t)1 << 40)
        return 0;
    return (size_t)zq::packed_weights_bytes(N, K);
}

ZQ_API zq_status zq_pack_weights(const int8_t *Wq, int64_t N, int64_t K, int8_t *Wp,
                                 hipStream_t stream)
{
    if (!Wq || !Wp)
        return ZQ_ERR_NULL;
    if (zq_packed_weights_bytes(N, K) == 0)
        return ZQ_ERR_SHAPE;
    if (!aligned16(Wq) || !aligned16(Wp))
        return ZQ_ERR_ALIGN;
    if (hip_error_pending())
        return ZQ_ERR_HIP;
    return map_hip(zq::launch_pack_weights(Wq, N, K, Wp, stream));
}

ZQ_API zq_status zq_w8a8_gemm_dequant_packed(const int8_t *Xq, const float *x_scales,
                                             const int8_t *Wp, const float *w_scales,
                                             int64_t group_rows, const float *bias, zq_act act,
                                             int64_t M, int64_t N, int64_t K, void *Y,
                                             zq_dtype y_dtype, hipStream_t stream)
{
    zq_status st = check_gemm(Xq, x_scales, Wp, w_scales, group_rows, act, M, N, K, Y, y_dtype,
                              bias);
    if (st != ZQ_OK)
        return st;
    if (M > kSkinnyMaxM)
        return ZQ_ERR_SHAPE;
    if (hip_error_pending())
        return ZQ_ERR_HIP;
    return map_hip(zq::launch_gemm_skinny_packed(Xq, x_scales, Wp, w_scales, group_rows, bias,
                                                 (int)act, M, N, K, Y, y_dtype == ZQ_I32,
                                                 stream));
}

// Workspace of zq_linear_w8a8_unfused: y fp16 [M*K] | codes [M*K] | scales [M] |
// accumulators int32 [M*N], each part starting on a 256-byte boundary.
ZQ_API size_t zq_linear_unfused_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    if (M < 1 || N < 1 || !k_ok(K) || M > INT32_MAX || N > INT32_MAX ||
        M * K > (int64_t)1 << 40 || M * N > (int64_t)1 << 38)
        return 0;
    return round_up(2 * (size_t)(M * K), 256) + round_up((size_t)(M * K), 256) +
           round_up(4 * (size_t)M, 256) + round_up(4 * (size_t)(M * N), 256);
}

ZQ_API zq_status zq_linear_w8a8_unfused(const void *X, zq_dtype x_dtype, zq_pre pre,
                                        const float *gamma, const float *beta, float eps,
                                        const int8_t *Wq, const float *w_scales,
                                        int64_t group_rows, const float *bias, zq_act act,
                                        int64_t M, int64_t N, int64_t K, void *workspace,
                                        size_t workspace_bytes, void *Y, hipStream_t stream)
{
    if (!X || !Wq || !w_scales || !Y)
        return ZQ_ERR_NULL;
    if (!workspace)
        return ZQ_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return ZQ_ERR_ALIGN;
    const size_t need = zq_linear_unfused_workspace_bytes(M, N, K);
    const size_t mk = (size_t)(M > 0 && K > 0 ? M * K : 0);
    char *ws = static_cast<char *>(workspace);
    _Float16 *y16 = reinterpret_cast<_Float16 *>(ws);
    int8_t *Xq = reinterpret_cast<int8_t *>(ws + round_up(2 * mk, 256));
    float *x_scales = reinterpret_cast<float *>(ws + round_up(2 * mk, 256) + round_up(mk, 256));
    int32_t *acc = reinterpret_cast<int32_t *>(ws + round_up(2 * mk, 256) + round_up(mk, 256) +
                                               round_up(4 * (size_t)(M > 0 ? M : 0), 256));
    zq_status st = check_prologue(X, x_dtype, M, K, pre, gamma, beta, Xq, x_scales);
    if (st != ZQ_OK)
        return st;
    st = check_gemm(Xq, x_scales, Wq, w_scales, group_rows, act, M, N, K, Y, ZQ_F16, bias);
    if (st != ZQ_OK)
        return st;
    if (need == 0)
        return ZQ_ERR_SHAPE;
    if (workspace_bytes < need)
        return ZQ_ERR_WORKSPACE;
    if (hip_error_pending())
        return ZQ_ERR_HIP;
    st = map_hip(zq::launch_ln_to_f16(X, x_dtype == ZQ_F16, M, K, (int)pre,
                                      pre == ZQ_PRE_LAYERNORM ? gamma : nullptr,
                                      pre == ZQ_PRE_LAYERNORM ? beta : nullptr, eps, y16, stream));
    if (st != ZQ_OK)
        return st;
    st = map_hip(zq::launch_ln_quant(y16, true, M, K, ZQ_PRE_NONE, nullptr, nullptr, eps, Xq,
                                     x_scales, stream));
    if (st != ZQ_OK)
        return st;
    st = gemm_dispatch(Xq, nullptr, Wq, nullptr, group_rows, nullptr, ZQ_ACT_NONE, M, N, K, acc,
                       ZQ_I32, ZQ_PATH_AUTO, stream);
    if (st != ZQ_OK)
        return st;
    return map_hip(zq::launch_dequant(acc, x_scales, w_scales, group_rows, bias, (int)act, M, N, Y,
                                      stream));
}

namespace {
// Column groups of H's partial row maxima: at most F / 16 + 2 for either GEMM.
int64_t ffn_row_groups_max(int64_t F)
{
    return F / 16 + 2;
}
}  // namespace

// Workspace of zq_ffn_w8a8: codes1 [M*K] | scales1 [M] | H fp16 [M*F] |
// partial row maxima fp32 [M * (F/16 + 2)] | codes2 [M*F] | scales2 [M], each part
// starting on a 256-byte boundary.
ZQ_API size_t zq_ffn_workspace_bytes(int64_t M, int64_t K, int64_t F)
{
    if (M < 1 || !k_ok(K) || !k_ok(F) || M > INT32_MAX || M * K > (int64_t)1 << 40 ||
        M * F > (int64_t)1 << 39)
        return 0;
    const size_t m = (size_t)M;
    return round_up(m * K, 256) + round_up(4 * m, 256) + round_up(2 * m * F, 256) +
           round_up(4 * m * (size_t)ffn_row_groups_max(F), 256) + round_up(m * F, 256) +
           round_up(4 * m, 256);
}

ZQ_API zq_status zq_ffn_w8a8(const void *X, zq_dtype x_dtype, const float *gamma,
                             const float *beta, float eps, const int8_t *W1q,
                             const float *w1_scales, int64_t group_rows1, const float *bias1,
                             const int8_t *W2q, const float *w2_scales, int64_t group_rows2,
                             const float *bias2, int64_t M, int64_t K, int64_t F,
                             void *workspace, size_t workspace_bytes, void *Y,
                             hipStream_t stream)
{
    if (!X || !W1q || !w1_scales || !W2q || !w2_scales || !Y)
        return ZQ_ERR_NULL;
    if (!workspace)
        return ZQ_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return ZQ_ERR_ALIGN;
    const size_t need = zq_ffn_workspace_bytes(M, K, F);
    const size_t m = (size_t)(M > 0 ? M : 0);
    const size_t mk = m * (size_t)(K > 0 ? K : 0), mf = m * (size_t)(F > 0 ? F : 0);
    char *ws = static_cast<char *>(workspace);
    size_t off = 0;
    int8_t *Xq1 = reinterpret_cast<int8_t *>(ws + off);
    off += round_up(mk, 256);
    float *sx1 = reinterpret_cast<float *>(ws + off);
    off += round_up(4 * m, 256);
    _Float16 *H = reinterpret_cast<_Float16 *>(ws + off);
    off += round_up(2 * mf, 256);
    float *part = reinterpret_cast<float *>(ws + off);
    off += round_up(4 * m * (size_t)(F > 0 ? ffn_row_groups_max(F) : 0), 256);
    int8_t *Xq2 = reinterpret_cast<int8_t *>(ws + off);
    off += round_up(mf, 256);
    float *sx2 = reinterpret_cast<float *>(ws + off);
    zq_status st = check_prologue(X, x_dtype, M, K, ZQ_PRE_LAYERNORM, gamma, beta, Xq1, sx1);
    if (st != ZQ_OK)
        return st;
    st = check_gemm(Xq1, sx1, W1q, w1_scales, group_rows1, ZQ_ACT_GELU, M, F, K, H, ZQ_F16, bias1);
    if (st != ZQ_OK)
        return st;
    st = check_gemm(Xq2, sx2, W2q, w2_scales, group_rows2, ZQ_ACT_NONE, M, K, F, Y, ZQ_F16, bias2);
    if (st != ZQ_OK)
        return st;
    if (need == 0)
        return ZQ_ERR_SHAPE;
    if (workspace_bytes < need)
        return ZQ_ERR_WORKSPACE;
    if (hip_error_pending())
        return ZQ_ERR_HIP;
    // FFN-up: LN + quantize ...
    st = map_hip(zq::launch_ln_quant(X, x_dtype == ZQ_F16, M, K, ZQ_PRE_LAYERNORM, gamma, beta,
                                     eps, Xq1, sx1, stream));
    if (st != ZQ_OK)
        return st;
    // ... GEMM + bias + GeLU, whose epilogue also writes partial maxima of |H[m, :]| ...
    const bool skinny = M <= kSkinnyMaxM;
    const int64_t groups = skinny ? zq::gemm_skinny_row_groups(F) : zq::gemm_tiled_row_groups(M, F);
    if (groups > ffn_row_groups_max(F))
        return ZQ_ERR_UNSUPPORTED;  // not reached: every column group has at least 16 columns
    if (skinny)
        st = map_hip(zq::launch_gemm_skinny(Xq1, sx1, W1q, w1_scales, group_rows1, bias1,
                                            ZQ_ACT_GELU, M, F, K, H, false, stream, part));
    else
        st = map_hip(zq::launch_gemm_tiled(Xq1, sx1, W1q, w1_scales, group_rows1, bias1,
                                           ZQ_ACT_GELU, M, F, K, H, false, stream, part));
    if (st != ZQ_OK)
        return st;
    // FFN-down: quantize H from the partial maxima, then GEMM + bias.
    st = map_hip(zq::launch_quant_rows_part(H, M, F, part, groups, Xq2, sx2, stream));
    if (st != ZQ_OK)
        return st;
    return gemm_dispatch(Xq2, sx2, W2q, w2_scales, group_rows2, bias2, ZQ_ACT_NONE, M, K, F, Y,
                         ZQ_F16, ZQ_PATH_AUTO, stream);
}

// ---- FP8 variant (OCP E4M3 codes, power-of-two scales) ----

ZQ_API zq_status zq_quantize_weights_grouped_fp8(const void *W, zq_dtype w_dtype,
                                                 const float *smooth, int64_t N, int64_t K,
                                                 int64_t group_rows, uint8_t *Wq8,
                                                 float *w_scales, hipStream_t stream)
{
    if (!W || !Wq8 || !w_scales)
        return ZQ_ERR_NULL;
    if (w_dtype != ZQ_F32 && w_dtype != ZQ_F16)
        return ZQ_ERR_DTYPE;
    if (N < 1 || !k_ok(K) || group_rows < 1 || N % group_rows != 0 || N > INT32_MAX ||
        N * K > (int64_t)1 << 40)
        return ZQ_ERR_SHAPE;
    if (!aligned16(W) || !aligned16(Wq8))
        return ZQ_ERR_ALIGN;
    if (hip_error_pending())
        return ZQ_ERR_HIP;
    return map_hip(zq::launch_quantize_weights(W, w_dtype == ZQ_F16, smooth, N, K, group_rows,
                                               reinterpret_cast<int8_t *>(Wq8), w_scales, stream,
                                               true));
}

ZQ_API zq_status zq_ln_quant_per_token_fp8(const void *X, zq_dtype x_dtype, int64_t M, int64_t K,
                                           zq_pre pre, const float *gamma, const float *beta,
                                           float eps, uint8_t *Xq8, float *x_scales,
                                           hipStream_t stream)
{
    int8_t *Xq = reinterpret_cast<int8_t *>(Xq8);
    zq_status st = check_prologue(X, x_dtype, M, K, pre, gamma, beta, Xq, x_scales);
    if (st != ZQ_OK)
        return st;
    if (hip_error_pending())
        return ZQ_ERR_HIP;
    return map_hip(zq::launch_ln_quant(X, x_dtype == ZQ_F16, M, K, (int)pre,
                                       pre == ZQ_PRE_LAYERNORM ? gamma : nullptr,
                                       pre == ZQ_PRE_LAYERNORM ? beta : nullptr, eps, Xq,
                                       x_scales, stream, true));
}

namespace {

zq_status fp8_gemm(const uint8_t *Xq8, const float *x_scales, const uint8_t *Wq8,
                   const float *w_scales, int64_t G, const float *bias, zq_act act, int64_t M,
                   int64_t N, int64_t K, void *Y, zq_dtype y_dtype, bool packed,
                   hipStream_t stream)
{
    const int8_t *Xq = reinterpret_cast<const int8_t *>(Xq8);
    const int8_t *Wq = reinterpret_cast<const int8_t *>(Wq8);
    const bool raw = y_dtype == ZQ_F32;
    if (packed || M <= kSkinnyMaxM)
        return map_hip(zq::launch_gemm_skinny_fp8(Xq, x_scales, Wq, w_scales, G, bias, (int)act,
                                                  M, N, K, Y, raw, packed, stream));
    return map_hip(zq::launch_gemm_tiled_fp8(Xq, x_scales, Wq, w_scales, G, bias, (int)act, M, N,
                                             K, Y, raw, stream));
}

zq_status check_fp8_gemm(const uint8_t *Xq8, const float *x_scales, const uint8_t *Wq8,
                         const float *w_scales, int64_t G, zq_act act, int64_t M, int64_t N,
                         int64_t K, const void *Y, zq_dtype y_dtype, const float *bias)
{
    if (y_dtype != ZQ_F16 && y_dtype != ZQ_F32)
        return ZQ_ERR_DTYPE;
    // The shape, alignment and pointer rules are those of the int8 GEMM (the
    // raw fp32 accumulators take the place of its int32 test mode).
    return check_gemm(reinterpret_cast<const int8_t *>(Xq8), x_scales,
                      reinterpret_cast<const int8_t *>(Wq8), w_scales, G, act, M, N, K, Y,
                      y_dtype == ZQ_F32 ? ZQ_I32 : ZQ_F16, bias);
}

}  // namespace

ZQ_API zq_status zq_fp8_gemm_dequant(const uint8_t *Xq8, const float *x_scales,
                                     const uint8_t *Wq8, const float *w_scales,
                                     int64_t group_rows, const float *bias, zq_act act,
                                     int64_t M, int64_t N, int64_t K, void *Y, zq_dtype y_dtype,
                                     hipStream_t stream)
{
    zq_status st = check_fp8_gemm(Xq8, x_scales, Wq8, w_scales, group_rows, act, M, N, K, Y,
                                  y_dtype, bias);
    if (st != ZQ_OK)
        return st;
    if (hip_error_pending())
        return ZQ_ERR_HIP;
    return fp8_gemm(Xq8, x_scales, Wq8, w_scales, group_rows, bias, act, M, N, K, Y, y_dtype,
                    false, stream);
}

namespace {

zq_status linear_fp8_impl(const void *X, zq_dtype x_dtype, zq_pre pre, const float *gamma,
                          const float *beta, float eps, const uint8_t *Wq8,
                          const float *w_scales, int64_t group_rows, const float *bias,
                          zq_act act, int64_t M, int64_t N, int64_t K, void *workspace,
                          size_t workspace_bytes, void *Y, bool packed, hipStream_t stream)
{
    if (!X || !Wq8 || !w_scales || !Y)
        return ZQ_ERR_NULL;
    if (!workspace)
        return ZQ_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return ZQ_ERR_ALIGN;
    const size_t need = zq_linear_workspace_bytes(M, K);
    const size_t codes_bytes = round_up((size_t)(M > 0 && K > 0 ? M * K : 0), 256);
    uint8_t *Xq8 = static_cast<uint8_t *>(workspace);
    float *x_scales = reinterpret_cast<float *>(static_cast<char *>(workspace) + codes_bytes);
    zq_status st = check_prologue(X, x_dtype, M, K, pre, gamma, beta,
                                  reinterpret_cast<int8_t *>(Xq8), x_scales);
    if (st != ZQ_OK)
        return st;
    st = check_fp8_gemm(Xq8, x_scales, Wq8, w_scales, group_rows, act, M, N, K, Y, ZQ_F16, bias);
    if (st != ZQ_OK)
        return st;
    if (packed && M > kSkinnyMaxM)
        return ZQ_ERR_SHAPE;
    if (workspace_bytes < need)
        return ZQ_ERR_WORKSPACE;
    if (hip_error_pending())
        return ZQ_ERR_HIP;
    st = map_hip(zq::launch_ln_quant(X, x_dtype == ZQ_F16, M, K, (int)pre,
                                     pre == ZQ_PRE_LAYERNORM ? gamma : nullptr,
                                     pre == ZQ_PRE_LAYERNORM ? beta : nullptr, eps,
                                     reinterpret_cast<int8_t *>(Xq8), x_scales, stream, true));
    if (st != ZQ_OK)
        return st;
    return fp8_gemm(Xq8, x_scales, Wq8, w_scales, group_rows, bias, act, M, N, K, Y, ZQ_F16,
                    packed, stream);
}

}  // namespace

ZQ_API zq_status zq_linear_w8a8_fp8(const void *X, zq_dtype x_dtype, zq_pre pre,
                                    const float *gamma, const float *beta, float eps,
                                    const uint8_t *Wq8, const float *w_scales, int64_t group_rows,
                                    const float *bias, zq_act act, int64_t M, int64_t N,
                                    int64_t K, void *workspace, size_t workspace_bytes, void *Y,
                                    hipStream_t stream)
{
    return linear_fp8_impl(X, x_dtype, pre, gamma, beta, eps, Wq8, w_scales, group_rows, bias,
                           act, M, N, K, workspace, workspace_bytes, Y, false, stream);
}

ZQ_API zq_status zq_linear_w8a8_fp8_packed(const void *X, zq_dtype x_dtype, zq_pre pre,
                                           const float *gamma, const float *beta, float eps,
                                           const uint8_t *Wp8, const float *w_scales,
                                           int64_t group_rows, const float *bias, zq_act act,
                                           int64_t M, int64_t N, int64_t K, void *workspace,
                                           size_t workspace_bytes, void *Y, hipStream_t stream)
{
    return linear_fp8_impl(X, x_dtype, pre, gamma, beta, eps, Wp8, w_scales, group_rows, bias,
                           act, M, N, K, workspace, workspace_bytes, Y, true, stream);
}

ZQ_API size_t zq_smoothquant_workspace_bytes(int64_t M, int64_t K)
{
    if (M < 1 || !k_ok(K) || M > INT32_MAX)
        return 0;
    return round_up(8 * (size_t)M + 8 * (size_t)K, 256);
}

ZQ_API zq_status zq_smoothquant_factors(const void *X, zq_dtype x_dtype, int64_t M, int64_t K,
                                        float eps, const void *W, zq_dtype w_dtype, int64_t N,
                                        const float *gamma, const float *beta, float *smooth,
                                        float *gamma_out, float *beta_out, void *workspace,
                                        size_t workspace_bytes, hipStream_t stream)
{
    if (!X || !W || !smooth || !gamma_out || !beta_out)
        return ZQ_ERR_NULL;
    if ((x_dtype != ZQ_F16 && x_dtype != ZQ_F32) || (w_dtype != ZQ_F16 && w_dtype != ZQ_F32))
        return ZQ_ERR_DTYPE;
    if (M < 1 || N < 1 || !k_ok(K) || M > INT32_MAX || N > INT32_MAX ||
        M * K > (int64_t)1 << 40 || N * K > (int64_t)1 << 40)
        return ZQ_ERR_SHAPE;
    if (!aligned16(X) || !aligned16(W))
        return ZQ_ERR_ALIGN;
    if (!workspace || workspace_bytes < zq_smoothquant_workspace_bytes(M, K))
        return ZQ_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return ZQ_ERR_ALIGN;
    if (hip_error_pending())
        return ZQ_ERR_HIP;
    return map_hip(zq::launch_smooth_factors(X, x_dtype == ZQ_F16, M, K, eps, W, w_dtype == ZQ_F16,
                                             N, gamma, beta, smooth, gamma_out, beta_out,
                                             workspace, stream));
}

// ---- Mixed-precision decomposition (outlier columns in fp16) ----

namespace {
// Few tokens: the weight-streaming kernel; otherwise the tiled one.
zq_status gemm_decomp_dispatch(const int8_t *Xq, const float *x_scales, const int8_t *Wq,
                               const float *w_scales, int64_t G, const float *bias, zq_act act,
                               int64_t M, int64_t N, int64_t K, const int32_t *cols,
                               const _Float16 *XO, const _Float16 *W16t, void *Y,
                               hipStream_t stream)
{
    if (M <= kSkinnyMaxM)
        return map_hip(zq::launch_gemm_skinny_decomp(Xq, x_scales, Wq, w_scales, G, bias, (int)act,
                                                     M, N, K, cols, XO, W16t, Y, stream));
    return map_hip(zq::launch_gemm_tiled_decomp(Xq, x_scales, Wq, w_scales, G, bias, (int)act, M,
                                                N, K, cols, XO, W16t, Y, stream));
}
}  // namespace

ZQ_API zq_status zq_pack_outlier_weights(const void *W, zq_dtype w_dtype, int64_t N, int64_t K,
                                         void *W16t, hipStream_t stream)
{
    if (!W || !W16t)
        return ZQ_ERR_NULL;
    if (w_dtype != ZQ_F32 && w_dtype != ZQ_F16)
        return ZQ_ERR_DTYPE;
    if (N < 1 || !k_ok(K) || N > INT32_MAX || N * K > (int64_t)1 << 40)
        return ZQ_ERR_SHAPE;
    if (!aligned16(W) || !aligned16(W16t))
        return ZQ_ERR_ALIGN;
    if (hip_error_pending())
        return ZQ_ERR_HIP;
    return map_hip(zq::launch_pack_outlier_weights(W, w_dtype == ZQ_F16, N, K,
                                                   static_cast<_Float16 *>(W16t), stream));
}

ZQ_API zq_status zq_outlier_columns(const void *X, zq_dtype x_dtype, int64_t M, int64_t K,
                                    zq_pre pre, const float *gamma, const float *beta, float eps,
                                    float alpha, int32_t *slot, int32_t *cols, hipStream_t stream)
{
    if (!slot || !cols)
        return ZQ_ERR_NULL;
    // The prologue's checks; the codes and scales pointers it wants are not used here.
    zq_status st = check_prologue(X, x_dtype, M, K, pre, gamma, beta,
                                  reinterpret_cast<const int8_t *>(slot),
                                  reinterpret_cast<const float *>(slot));
    if (st != ZQ_OK)
        return st;
    if (!aligned16(slot))
        return ZQ_ERR_ALIGN;
    if (hip_error_pending())
        return ZQ_ERR_HIP;
    return map_hip(zq::launch_outlier_columns(X, x_dtype == ZQ_F16, M, K, (int)pre,
                                              pre == ZQ_PRE_LAYERNORM ? gamma : nullptr,
                                              pre == ZQ_PRE_LAYERNORM ? beta : nullptr, eps,
                                              alpha, slot, cols, stream));
}

ZQ_API zq_status zq_ln_quant_decomp(const void *X, zq_dtype x_dtype, int64_t M, int64_t K,
                                    zq_pre pre, const float *gamma, const float *beta, float eps,
                                    const int32_t *slot, int8_t *Xq, float *x_scales, void *XO,
                                    hipStream_t stream)
{
    if (!slot || !XO)
        return ZQ_ERR_NULL;
    zq_status st = check_prologue(X, x_dtype, M, K, pre, gamma, beta, Xq, x_scales);
    if (st != ZQ_OK)
        return st;
    if (!aligned16(slot) || !aligned16(XO))
        return ZQ_ERR_ALIGN;
    if (hip_error_pending())
        return ZQ_ERR_HIP;
    return map_hip(zq::launch_ln_quant_decomp(X, x_dtype == ZQ_F16, M, K, (int)pre,
                                              pre == ZQ_PRE_LAYERNORM ? gamma : nullptr,
                                              pre == ZQ_PRE_LAYERNORM ? beta : nullptr, eps, slot,
                                              Xq, x_scales, static_cast<_Float16 *>(XO), stream));
}

ZQ_API zq_status zq_w8a8_gemm_decomp(const int8_t *Xq, const float *x_scales, const int8_t *Wq,
                                     const float *w_scales, int64_t group_rows,
                                     const int32_t *cols, const void *XO, const void *W16t,
                                     const float *bias, zq_act act, int64_t M, int64_t N,
                                     int64_t K, void *Y, hipStream_t stream)
{
    if (!cols || !XO || !W16t)
        return ZQ_ERR_NULL;
    zq_status st = check_gemm(Xq, x_scales, Wq, w_scales, group_rows, act, M, N, K, Y, ZQ_F16,
                              bias);
    if (st != ZQ_OK)
        return st;
    if (!aligned16(XO) || !aligned16(W16t))
        return ZQ_ERR_ALIGN;
    if (hip_error_pending())
        return ZQ_ERR_HIP;
    return gemm_decomp_dispatch(Xq, x_scales, Wq, w_scales, group_rows, bias, act, M, N, K, cols,
                                static_cast<const _Float16 *>(XO),
                                static_cast<const _Float16 *>(W16t), Y, stream);
}

// Workspace of zq_linear_w8a8_decomp: slot int32 [K] | cols int32 [K + 1] |
// codes [M*K] | scales [M] | XO fp16 [M*K], each part starting on a 256-byte boundary.
ZQ_API size_t zq_linear_decomp_workspace_bytes(int64_t M, int64_t K)
{
    if (M < 1 || !k_ok(K) || M > INT32_MAX || M * K > (int64_t)1 << 40)
        return 0;
    return round_up(4 * (size_t)K, 256) + round_up(4 * (size_t)(K + 1), 256) +
           round_up((size_t)(M * K), 256) + round_up(4 * (size_t)M, 256) +
           round_up(2 * (size_t)(M * K), 256);
}

ZQ_API zq_status zq_linear_w8a8_decomp(const void *X, zq_dtype x_dtype, zq_pre pre,
                                       const float *gamma, const float *beta, float eps,
                                       float alpha, const int8_t *Wq, const float *w_scales,
                                       int64_t group_rows, const void *W16t, const float *bias,
                                       zq_act act, int64_t M, int64_t N, int64_t K,
                                       void *workspace, size_t workspace_bytes, void *Y,
                                       hipStream_t stream)
{
    if (!X || !Wq || !w_scales || !W16t || !Y)
        return ZQ_ERR_NULL;
    if (!workspace)
        return ZQ_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return ZQ_ERR_ALIGN;
    const size_t need = zq_linear_decomp_workspace_bytes(M, K);
    const size_t kk = (size_t)(K > 0 ? K : 0);
    const size_t mk = (size_t)(M > 0 && K > 0 ? M * K : 0);
    char *ws = static_cast<char *>(workspace);
    size_t off = 0;
    int32_t *slot = reinterpret_cast<int32_t *>(ws + off);
    off += round_up(4 * kk, 256);
    int32_t *cols = reinterpret_cast<int32_t *>(ws + off);
    off += round_up(4 * (kk + 1), 256);
    int8_t *Xq = reinterpret_cast<int8_t *>(ws + off);
    off += round_up(mk, 256);
    float *x_scales = reinterpret_cast<float *>(ws + off);
    off += round_up(4 * (size_t)(M > 0 ? M : 0), 256);
    _Float16 *XO = reinterpret_cast<_Float16 *>(ws + off);
    zq_status st = check_prologue(X, x_dtype, M, K, pre, gamma, beta, Xq, x_scales);
    if (st != ZQ_OK)
        return st;
    st = check_gemm(Xq, x_scales, Wq, w_scales, group_rows, act, M, N, K, Y, ZQ_F16, bias);
    if (st != ZQ_OK)
        return st;
    if (!aligned16(W16t))
        return ZQ_ERR_ALIGN;
    if (workspace_bytes < need)
        return ZQ_ERR_WORKSPACE;
    const float *g = pre == ZQ_PRE_LAYERNORM ? gamma : nullptr;
    const float *b = pre == ZQ_PRE_LAYERNORM ? beta : nullptr;
    if (hip_error_pending())
        return ZQ_ERR_HIP;
    st = map_hip(zq::launch_outlier_columns(X, x_dtype == ZQ_F16, M, K, (int)pre, g, b, eps, alpha,
                                            slot, cols, stream));
    if (st != ZQ_OK)
        return st;
    st = map_hip(zq::launch_ln_quant_decomp(X, x_dtype == ZQ_F16, M, K, (int)pre, g, b, eps, slot,
                                            Xq, x_scales, XO, stream));
    if (st != ZQ_OK)
        return st;
    return gemm_decomp_dispatch(Xq, x_scales, Wq, w_scales, group_rows, bias, act, M, N, K, cols,
                                XO, static_cast<const _Float16 *>(W16t), Y, stream);
}
