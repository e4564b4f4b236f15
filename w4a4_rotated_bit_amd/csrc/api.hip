// api.hip -- device entry points of the ConvRot C ABI (declared in
// include/convrot.h).  Each call checks its arguments on the host, checks that
// the current device is a gfx950, enqueues kernels on the caller's stream and
// returns; nothing here allocates, frees or synchronises.
#include <hip/hip_runtime.h>
#include <string.h>

#include <atomic>

#include "../../include/convrot.h"
#include "internal.h"
#include "kernels.h"
#include "layout.h"

using namespace convrot;

namespace {

// Per-device answer to "is this a gfx950?": 0 unknown, 1 yes, 2 no.
std::atomic<int> g_arch_ok[64];

int check_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return CONVROT_EHIP;
    if (dev >= 64) return CONVROT_EDEVICE;
    int known = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (known == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return CONVROT_EHIP;
        known = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_arch_ok[dev].store(known, std::memory_order_relaxed);
    }
    return known == 1 ? CONVROT_OK : CONVROT_EDEVICE;
}

int launched()
{
    return hipGetLastError() == hipSuccess ? CONVROT_OK : CONVROT_EHIP;
}

hipStream_t as_stream(void* s) { return (hipStream_t)s; }

int validate_rows_out(const void* X, int64_t rows, int64_t K, int g)
{
    int rc = check_shape(rows, K, g);
    if (rc) return rc;
    if (rows > 0 && (!X || !aligned(X, 16))) return CONVROT_EINVAL;
    return CONVROT_OK;
}

// want_fp6: also write the FP6 copy of the codes (when the GEMM that follows
// is unknown, or its plan reads that copy)
int enqueue_prepare_activations(const void* X, int64_t M, int64_t K, int g, void* ws, bool want_fp6, hipStream_t s)
{
    const int64_t Kr = rotated_width(K, g);
    PrepArgs a{};
    a.X = (const uint16_t*)X;
    a.ld = K;
    a.rows = M;
    a.rows_pad = round_up(M, kTileRows);
    a.K = Kr;
    a.K_pad = round_up(Kr, kTileK);
    a.out = (uint8_t*)ws + workspace_image_offset();
    a.out6 = act_has_fp6(M) && want_fp6 ? (uint8_t*)ws + workspace_image6_offset(M, Kr) : nullptr;
    a.scales = (float*)((uint8_t*)ws + workspace_sx_offset(M, Kr));
    a.rotated = nullptr;
    a.zero = (uint32_t*)ws;
    a.zero_count = 2 * kSplitCounters;
    launch_prep(g, OUT_IMAGE, a, s);
    return launched();
}

GemmArgs gemm_args(const void* ws, int64_t M, int64_t K, const void* image, const float* sw, const void* bias,
                   int64_t N, void* Y)
{
    GemmArgs a{};
    a.act = (const uint8_t*)ws + workspace_image_offset();
    a.wgt = (const uint8_t*)image;
    a.act6 = (const uint8_t*)ws + workspace_image6_offset(M, K);
    a.wgt6 = (const uint8_t*)image + weight_image6_offset(N, K);
    a.sx = (const float*)((const uint8_t*)ws + workspace_sx_offset(M, K));
    a.sw = sw;
    a.bias = (const uint16_t*)bias;
    a.out = Y;
    a.M = M;
    a.N = N;
    a.K = K;
    a.MT = (int)(round_up(M, kTileRows) / kTileRows);
    a.NT = (int)(round_up(N, kTileRows) / kTileRows);
    a.KB = (int)(round_up(K, kTileK) / kTileK);
    const GemmPlan plan = gemm_plan(M, N, K);
    a.shape = plan.shape;
    a.tiles_m = plan.tiles_m;
    a.tiles_n = plan.tiles_n;
    a.splits = plan.splits;
    a.counters = (uint32_t*)ws;
    a.partial = (int32_t*)((uint8_t*)ws + workspace_partial_offset(M, K));
    return a;
}

int enqueue_gemm(int out_mode, const void* ws, int64_t M, int64_t K, const void* image, const float* sw,
                 const void* bias, int64_t N, void* Y, hipStream_t s)
{
    launch_gemm(out_mode, gemm_args(ws, M, K, image, sw, bias, N, Y), s);
    return launched();
}

}  // namespace

extern "C" {

int convrot_prepare_weight(const void* W, int64_t N, int64_t K, int g, void* image, float* sw, void* stream)
{
    int rc = convrot_validate_weight(W, N, K, g, image, sw);
    if (rc || N == 0) return rc;
    if ((rc = check_device())) return rc;
    const int64_t Kr = rotated_width(K, g);
    PrepArgs a{};
    a.X = (const uint16_t*)W;
    a.ld = K;
    a.rows = N;
    a.rows_pad = round_up(N, kTileRows);
    a.K = Kr;
    a.K_pad = round_up(Kr, kTileK);
    a.out = (uint8_t*)image;
    a.out6 = (uint8_t*)image + weight_image6_offset(N, Kr);
    a.scales = sw;
    launch_prep(g, OUT_IMAGE, a, as_stream(stream));
    return launched();
}

int convrot_quantize_weight(const void* W, int64_t N, int64_t K, int g, uint8_t* qweight_nk, float* sw,
                            void* stream)
{
    int rc = convrot_validate_weight(W, N, K, g, qweight_nk, sw);
    if (rc || N == 0) return rc;
    if ((rc = check_device())) return rc;
    PrepArgs a{};
    a.X = (const uint16_t*)W;
    a.ld = K;
    a.rows = N;
    a.rows_pad = N;
    a.K = rotated_width(K, g);
    a.K_pad = a.K;
    a.out = qweight_nk;
    a.scales = sw;
    launch_prep(g, OUT_NK, a, as_stream(stream));
    return launched();
}

int convrot_repack_nk_to_image(const uint8_t* qweight_nk, int64_t N, int64_t K, void* image, void* stream)
{
    int rc = check_shape(N, K, 64);
    if (rc) return rc;
    if (N == 0) return CONVROT_OK;
    if (!qweight_nk || !image || !aligned(qweight_nk, 16) || !aligned(image, 16)) return CONVROT_EINVAL;
    if ((rc = check_device())) return rc;
    launch_repack_nk(qweight_nk, N, K, (uint8_t*)image, (uint8_t*)image + weight_image6_offset(N, K),
                     as_stream(stream));
    return launched();
}

int convrot_prepare_activations(const void* X, int64_t M, int64_t K, int g, void* ws, size_t ws_bytes,
                                void* stream)
{
    int rc = validate_rows_out(X, M, K, g);
    if (rc || M == 0) return rc;
    if (!ws || !aligned(ws, 16)) return CONVROT_EINVAL;
    if (ws_bytes < workspace_partial_offset(M, rotated_width(K, g))) return CONVROT_EWORKSPACE;
    if ((rc = check_device())) return rc;
    // the GEMM that will consume the workspace is not known: both copies
    return enqueue_prepare_activations(X, M, K, g, ws, true, as_stream(stream));
}

int convrot_gemm(const void* ws, size_t ws_bytes, int64_t M, int64_t K, const void* image, const float* sw,
                 const void* bias, int64_t N, void* Y, void* stream)
{
    // same checks as the linear, with the workspace standing in for X
    int rc = convrot_validate_linear(ws, M, K, image, sw, bias, N, 64, Y, ws, ws_bytes);
    if (rc || M == 0 || N == 0) return rc;
    if ((rc = check_device())) return rc;
    return enqueue_gemm(GEMM_OUT_BF16, ws, M, K, image, sw, bias, N, Y, as_stream(stream));
}

int convrot_linear(const void* X, int64_t M, int64_t K, const void* image, const float* sw, const void* bias,
                   int64_t N, int g, void* Y, void* ws, size_t ws_bytes, void* stream)
{
    int rc = convrot_validate_linear(X, M, K, image, sw, bias, N, g, Y, ws, ws_bytes);
    if (rc || M == 0 || N == 0) return rc;
    if ((rc = check_device())) return rc;
    hipStream_t s = as_stream(stream);
    const int64_t Kr = rotated_width(K, g);
    if (single_kernel_linear(M, Kr, g)) {
        // one kernel: each workgroup quantizes the few activation rows itself
        GemmArgs ga = gemm_args(ws, M, Kr, image, sw, bias, N, Y);
        PrepArgs pa{};
        pa.X = (const uint16_t*)X;
        pa.ld = K;
        pa.rows = M;
        pa.K = Kr;
        pa.K_pad = round_up(Kr, kTileK);
        pa.out = (uint8_t*)ws + workspace_image_offset();
        pa.scales = (float*)((uint8_t*)ws + workspace_sx_offset(M, Kr));
        launch_small_m(g, ga, pa, s);
        return launched();
    }
    const bool fp6 = gemm_shape_fp6(gemm_plan(M, N, Kr).shape);
    if ((rc = enqueue_prepare_activations(X, M, K, g, ws, fp6, s))) return rc;
    return enqueue_gemm(GEMM_OUT_BF16, ws, M, Kr, image, sw, bias, N, Y, s);
}

int convrot_linear_w4a16(const void* X, int64_t M, int64_t K, const void* image, const float* sw, const void* bias,
                         int64_t N, int g, void* Y, void* ws, size_t ws_bytes, void* stream)
{
    int rc = convrot_validate_linear_w4a16(X, M, K, image, sw, bias, N, g, Y, ws, ws_bytes);
    if (rc || M == 0 || N == 0) return rc;
    if ((rc = check_device())) return rc;
    hipStream_t s = as_stream(stream);
    const int64_t Kr = rotated_width(K, g);
    if (single_kernel_linear(M, Kr, g)) {
        // one kernel: each workgroup rotates the few activation rows itself
        GemmArgs ga = gemm_args(ws, M, Kr, image, sw, bias, N, Y);
        PrepArgs pa{};
        pa.X = (const uint16_t*)X;
        pa.ld = K;
        pa.rows = M;
        pa.K = Kr;
        pa.K_pad = round_up(Kr, kTileK);
        pa.out = (uint8_t*)ws;
        launch_small_w4a16(g, ga, pa, s);
        return launched();
    }
    // 1. the rotated activation rows, rounded to bf16, into the workspace
    PrepArgs a{};
    a.X = (const uint16_t*)X;
    a.ld = K;
    a.rows = M;
    a.rows_pad = M;
    a.K = Kr;
    a.K_pad = Kr;
    a.out = (uint8_t*)ws;
    launch_prep(g, OUT_ROTATED_BF16, a, s);
    if ((rc = launched())) return rc;
    // 2. their product with the weight image, scale and bias
    GemmArgs ga = gemm_args(ws, M, Kr, image, sw, bias, N, Y);
    launch_w4a16(ga, (const uint16_t*)ws, s);
    return launched();
}

int convrot_prepare_rows(const void* X, int64_t rows, int64_t K, int g, int8_t* codes, float* scales,
                         float* rotated, void* stream)
{
    int rc = validate_rows_out(X, rows, K, g);
    if (rc || rows == 0) return rc;
    if (!codes || !scales || !aligned(codes, 16) || (rotated && !aligned(rotated, 16))) return CONVROT_EINVAL;
    if ((rc = check_device())) return rc;
    PrepArgs a{};
    a.X = (const uint16_t*)X;
    a.ld = K;
    a.rows = rows;
    a.rows_pad = rows;
    a.K = rotated_width(K, g);
    a.K_pad = a.K;
    a.out = (uint8_t*)codes;
    a.scales = scales;
    a.rotated = rotated;
    launch_prep(g, OUT_ROWMAJOR, a, as_stream(stream));
    return launched();
}

int convrot_gemm_i32(const int8_t* qx, int64_t M, int64_t K, const void* image, int64_t N, int32_t* acc, void* ws,
                     size_t ws_bytes, void* stream)
{
    int rc = check_shape(M, K, 64);
    if (rc) return rc;
    if (N < 0 || N > kMaxRows) return CONVROT_EINVAL;
    if (M == 0 || N == 0) return CONVROT_OK;
    if (!qx || !image || !acc || !ws) return CONVROT_EINVAL;
    if (!aligned(qx, 16) || !aligned(image, 16) || !aligned(acc, 16) || !aligned(ws, 16)) return CONVROT_EINVAL;
    if (ws_bytes < workspace_bytes(M, K, N)) return CONVROT_EWORKSPACE;
    if ((rc = check_device())) return rc;
    hipStream_t s = as_stream(stream);
    uint8_t* image6 = act_has_fp6(M) ? (uint8_t*)ws + workspace_image6_offset(M, K) : nullptr;
    launch_act_relayout(qx, M, K, (uint8_t*)ws + workspace_image_offset(), image6, (uint32_t*)ws,
                        2 * kSplitCounters, s);
    if ((rc = launched())) return rc;
    return enqueue_gemm(GEMM_OUT_I32, ws, M, K, image, nullptr, nullptr, N, acc, s);
}

}  // extern "C"
