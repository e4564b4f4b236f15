// api.hip -- device entry points of the ConvRot C ABI (declared in
// include/convrot.h).  Each call checks its arguments on the host, checks that
// the current device is a gfx950, enqueues kernels on the caller's stream and
// returns; nothing here allocates, frees or synchronises.  The one piece of
// state is the allocation-free linear's workspace: a file-scope device array
// (each GPU holds its own copy for the life of the process) whose address is
// looked up once per device.
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

// The workspace of convrot_linear_noalloc.  In host code `scratch` names a
// host-side stand-in, not device memory: only the per-device address from
// hipGetSymbolAddress (scratch_ptr) is ever passed to a kernel.
constexpr size_t kScratchBytes = (size_t)CONVROT_NOALLOC_MAX_WORKSPACE;
__device__ __align__(256) uint8_t scratch[kScratchBytes];
std::atomic<void*> g_scratch_ptr[64];

// This device's copy of `scratch`, looked up on the first call on the device
// (the device is current), or nullptr when the lookup fails.
void* scratch_ptr()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);  // racing first calls store the same address
    return p;
}

int validate_rows_out(const void* X, int64_t rows, int64_t K, int g)
{
    int rc = check_shape(rows, K, g);
    if (rc) return rc;
    if (rows > 0 && (!X || !aligned(X, 16))) return CONVROT_EINVAL;
    return CONVROT_OK;
}

// want4 / want6: write the INT4 activation image / its FP6 copy (both when
// the GEMM that follows is unknown; otherwise the one its plan reads).  The
// FP6 copy exists only when act_has_fp6(M, image_has_fp6(g)).  Clears the
// split-K counters and the status word.
// x_stream: read X with non-temporal loads.  The linear asks for it when a
// block tile other than the FP6 256 x 256 one follows: X (9.4 MB at the
// FLUX shapes, 37.7 MB for the down-projection) then does not stay in the
// caches, which otherwise slowed the GEMM launched right after (its weight
// stream's latency went up: the FP6 192 x 384 tile, whose two-stage ring
// looks ahead one stage only, took 44 instead of 36 us at 1536 x 12288).
int enqueue_prepare_activations(const void* X, int64_t M, int64_t K, int g, void* ws, bool want4, bool want6,
                                hipStream_t s, bool x_stream = false)
{
    const int64_t Kr = rotated_width(K, g);
    const bool fp6 = image_has_fp6(g);
    PrepArgs a{};
    a.X = (const uint16_t*)X;
    a.ld = K;
    a.rows = M;
    a.rows_pad = round_up(M, kTileRows);
    a.K = Kr;
    a.K_pad = round_up(Kr, kTileK);
    a.out6 = act_has_fp6(M, fp6) && want6 ? (uint8_t*)ws + workspace_image6_offset(M, Kr) : nullptr;
    a.out = want4 || !a.out6 ? (uint8_t*)ws + workspace_image_offset() : nullptr;
    a.scales = (float*)((uint8_t*)ws + workspace_sx_offset(M, Kr, fp6));
    a.rotated = nullptr;
    a.zero = (uint32_t*)ws;
    a.zero_count = kZeroWords;
    a.x_stream = x_stream ? 1 : 0;
    launch_prep(g, OUT_IMAGE, a, s);
    return launched();
}

// K: the code width.  fp6: the workspace layout has the FP6 activation part
// (and the weight image its FP6 copy).
GemmArgs gemm_args(const void* ws, int64_t M, int64_t K, const void* image, const float* sw, const void* bias,
                   int64_t N, void* Y, bool fp6, const GemmPlan& plan)
{
    GemmArgs a{};
    a.act = (const uint8_t*)ws + workspace_image_offset();
    a.wgt = (const uint8_t*)image;
    a.act6 = (const uint8_t*)ws + workspace_image6_offset(M, K);
    a.wgt6 = (const uint8_t*)image + weight_image6_offset(N, K);
    a.sx = (const float*)((const uint8_t*)ws + workspace_sx_offset(M, K, fp6));
    a.sw = sw;
    a.bias = (const uint16_t*)bias;
    a.out = Y;
    a.M = M;
    a.N = N;
    a.K = K;
    a.MT = (int)(round_up(M, kTileRows) / kTileRows);
    a.NT = (int)(round_up(N, kTileRows) / kTileRows);
    a.KB = (int)(round_up(K, kTileK) / kTileK);
    a.shape = plan.shape;
    a.tiles_m = plan.tiles_m;
    a.tiles_n = plan.tiles_n;
    a.splits = plan.splits;
    a.counters = (uint32_t*)ws;
    a.partial = (int32_t*)((uint8_t*)ws + workspace_partial_offset(M, K, fp6));
    a.status = (uint32_t*)((uint8_t*)ws + CONVROT_WORKSPACE_STATUS_OFFSET);
    a.spin_limit = kSplitSpinLimit;
    a.extra_wait = 0;
    return a;
}

GemmArgs gemm_args(const void* ws, int64_t M, int64_t K, const void* image, const float* sw, const void* bias,
                   int64_t N, void* Y, bool fp6)
{
    return gemm_args(ws, M, K, image, sw, bias, N, Y, fp6, gemm_plan(M, N, K, fp6));
}

int enqueue_gemm(int out_mode, const GemmArgs& a, hipStream_t s)
{
    // the split-K exchange has two counters per (tile, sub-block) in the
    // workspace's 2 kSplitCounters counter words; every plan stays inside
    if (a.splits > 1 && (int64_t)a.tiles_m * a.tiles_n * a.splits > kSplitCounters) return CONVROT_EINVAL;
    launch_gemm(out_mode, a, s);
    return launched();
}

// int8 codes [M][K] into the workspace's activation images (the FP6 one when
// fp6), clearing the counters and the status word
int enqueue_act_relayout(const int8_t* qx, int64_t M, int64_t K, void* ws, bool fp6, hipStream_t s)
{
    uint8_t* image6 = act_has_fp6(M, fp6) ? (uint8_t*)ws + workspace_image6_offset(M, K) : nullptr;
    launch_act_relayout(qx, M, K, (uint8_t*)ws + workspace_image_offset(), image6, (uint32_t*)ws, kZeroWords, s);
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
    a.out6 = image_has_fp6(g) ? (uint8_t*)image + weight_image6_offset(N, Kr) : nullptr;
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

static_assert(CONVROT_PROBE_FP6 == kProbeFp6 && CONVROT_PROBE_INT8 == kProbeInt8, "probe kinds of the header");

int convrot_matrix_core_probe_bytes(size_t* bytes_host)
{
    if (!bytes_host) return CONVROT_EINVAL;
    int rc = check_device();
    if (rc) return rc;
    *bytes_host = (size_t)probe_grid() * kProbeThreads * sizeof(float);
    return CONVROT_OK;
}

int convrot_matrix_core_probe(int kind, int iterations, float* out, size_t out_bytes, int64_t* mfma_count_host,
                              void* stream)
{
    if ((kind != kProbeFp6 && kind != kProbeInt8) || iterations < 1 || iterations > (1 << 24) || !mfma_count_host ||
        !out || !aligned(out, 4))
        return CONVROT_EINVAL;
    int rc = check_device();
    if (rc) return rc;
    if (out_bytes < (size_t)probe_grid() * kProbeThreads * sizeof(float)) return CONVROT_EWORKSPACE;
    *mfma_count_host = probe_grid() * (kProbeThreads / 64) * (int64_t)iterations * 4;
    launch_mfma_probe(kind, iterations, out, as_stream(stream));
    return launched();
}

int convrot_repack_nk_to_image(const uint8_t* qweight_nk, int64_t N, int64_t K, int g, void* image, void* stream)
{
    int rc = check_shape(N, K, g);
    if (rc) return rc;
    if (N == 0) return CONVROT_OK;
    if (!qweight_nk || !image || !aligned(qweight_nk, 16) || !aligned(image, 16)) return CONVROT_EINVAL;
    if ((rc = check_device())) return rc;
    const int64_t Kr = rotated_width(K, g);
    launch_repack_nk(qweight_nk, N, Kr, (uint8_t*)image,
                     image_has_fp6(g) ? (uint8_t*)image + weight_image6_offset(N, Kr) : nullptr, as_stream(stream));
    return launched();
}

int convrot_prepare_activations(const void* X, int64_t M, int64_t K, int g, void* ws, size_t ws_bytes,
                                void* stream)
{
    int rc = validate_rows_out(X, M, K, g);
    if (rc || M == 0) return rc;
    if (!ws || !aligned(ws, 16)) return CONVROT_EINVAL;
    if (ws_bytes < workspace_partial_offset(M, rotated_width(K, g), image_has_fp6(g))) return CONVROT_EWORKSPACE;
    if ((rc = check_device())) return rc;
    // the GEMM that will consume the workspace is not known: both copies
    return enqueue_prepare_activations(X, M, K, g, ws, true, true, as_stream(stream));
}

int convrot_gemm(const void* ws, size_t ws_bytes, int64_t M, int64_t K, const void* image, const float* sw,
                 const void* bias, int64_t N, int g, void* Y, void* stream)
{
    // same checks as the linear, with the workspace standing in for X
    int rc = convrot_validate_linear(ws, M, K, image, sw, bias, N, g, Y, ws, ws_bytes);
    if (rc || M == 0 || N == 0) return rc;
    if ((rc = check_device())) return rc;
    const int64_t Kr = rotated_width(K, g);
    return enqueue_gemm(GEMM_OUT_BF16, gemm_args(ws, M, Kr, image, sw, bias, N, Y, image_has_fp6(g)),
                        as_stream(stream));
}

// convrot_linear after its checks: ws is a workspace of at least
// convrot_workspace_bytes(M, K, N, g) bytes
static int enqueue_linear(const void* X, int64_t M, int64_t K, const void* image, const float* sw, const void* bias,
                          int64_t N, int g, void* Y, void* ws, hipStream_t s)
{
    const int64_t Kr = rotated_width(K, g);
    const bool fp6 = image_has_fp6(g);
    if (single_kernel_linear(M, Kr, g)) {
        // one kernel: each workgroup quantizes the few activation rows itself
        GemmArgs ga = gemm_args(ws, M, Kr, image, sw, bias, N, Y, fp6);
        PrepArgs pa{};
        pa.X = (const uint16_t*)X;
        pa.ld = K;
        pa.rows = M;
        pa.K = Kr;
        pa.K_pad = round_up(Kr, kTileK);
        pa.out = (uint8_t*)ws + workspace_image_offset();
        pa.scales = (float*)((uint8_t*)ws + workspace_sx_offset(M, Kr, fp6));
        launch_small_m(g, ga, pa, s);
        return launched();
    }
    const GemmPlan plan = gemm_plan(M, N, Kr, fp6);
    const bool fp6_plan = gemm_shape_fp6(plan.shape);  // the GEMM reads only the FP6 copy, else only the INT4 image
    const bool x_stream = M > kStreamMaxRows && plan.shape != 2;
    int rc = enqueue_prepare_activations(X, M, K, g, ws, !fp6_plan, fp6_plan, s, x_stream);
    if (rc) return rc;
    return enqueue_gemm(GEMM_OUT_BF16, gemm_args(ws, M, Kr, image, sw, bias, N, Y, fp6, plan), s);
}

int convrot_linear(const void* X, int64_t M, int64_t K, const void* image, const float* sw, const void* bias,
                   int64_t N, int g, void* Y, void* ws, size_t ws_bytes, void* stream)
{
    int rc = convrot_validate_linear(X, M, K, image, sw, bias, N, g, Y, ws, ws_bytes);
    if (rc || M == 0 || N == 0) return rc;
    if ((rc = check_device())) return rc;
    return enqueue_linear(X, M, K, image, sw, bias, N, g, Y, ws, as_stream(stream));
}

int convrot_linear_noalloc(const void* X, int64_t M, int64_t K, const void* image, const float* sw,
                           const void* bias, int64_t N, int g, void* Y, void* stream)
{
    // the checks of convrot_linear, with a stand-in for the workspace (any
    // non-null aligned value) and the size of the static one
    static const uint8_t kStandIn alignas(256) = 0;
    int rc = convrot_validate_linear(X, M, K, image, sw, bias, N, g, Y, &kStandIn, kScratchBytes);
    if (rc || M == 0 || N == 0) return rc;
    if ((rc = check_device())) return rc;
    void* ws = scratch_ptr();
    if (!ws) return CONVROT_EHIP;
    return enqueue_linear(X, M, K, image, sw, bias, N, g, Y, ws, as_stream(stream));
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
        GemmArgs ga = gemm_args(ws, M, Kr, image, sw, bias, N, Y, false);
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
    GemmArgs ga = gemm_args(ws, M, Kr, image, sw, bias, N, Y, false);
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

static int check_gemm_i32(const int8_t* qx, int64_t M, int64_t K, const void* image, int64_t N, const int32_t* acc,
                          const void* ws)
{
    int rc = check_shape(M, K, 64);
    if (rc) return rc;
    if (N < 0 || N > kMaxRows) return CONVROT_EINVAL;
    if (M == 0 || N == 0) return CONVROT_OK;
    if (!qx || !image || !acc || !ws) return CONVROT_EINVAL;
    if (!aligned(qx, 16) || !aligned(image, 16) || !aligned(acc, 16) || !aligned(ws, 16)) return CONVROT_EINVAL;
    return CONVROT_OK;
}

int convrot_gemm_i32(const int8_t* qx, int64_t M, int64_t K, const void* image, int64_t N, int32_t* acc, void* ws,
                     size_t ws_bytes, void* stream)
{
    int rc = check_gemm_i32(qx, M, K, image, N, acc, ws);
    if (rc || M == 0 || N == 0) return rc;
    if (ws_bytes < workspace_bytes(M, K, N, true)) return CONVROT_EWORKSPACE;
    if ((rc = check_device())) return rc;
    hipStream_t s = as_stream(stream);
    if ((rc = enqueue_act_relayout(qx, M, K, ws, true, s))) return rc;
    return enqueue_gemm(GEMM_OUT_I32, gemm_args(ws, M, K, image, nullptr, nullptr, N, acc, true), s);
}

int convrot_gemm_i32_tiled(const int8_t* qx, int64_t M, int64_t K, const void* image, int64_t N, int32_t* acc,
                           int tile_m, int tile_n, int splits, int test_flags, void* ws, size_t ws_bytes,
                           void* stream)
{
    int rc = check_gemm_i32(qx, M, K, image, N, acc, ws);
    if (rc || M == 0 || N == 0) return rc;
    if (test_flags & ~CONVROT_TEST_SPLIT_TIMEOUT) return CONVROT_EINVAL;
    GemmPlan plan;
    const bool fp6 = gemm_shape_fp6(gemm_shape_of(tile_m, tile_n));
    if ((rc = check_forced_plan(M, K, N, tile_m, tile_n, splits, fp6, &plan))) return rc;
    if (ws_bytes < workspace_bytes_for(M, K, fp6, plan)) return CONVROT_EWORKSPACE;
    if ((rc = check_device())) return rc;
    hipStream_t s = as_stream(stream);
    if ((rc = enqueue_act_relayout(qx, M, K, ws, fp6, s))) return rc;
    GemmArgs a = gemm_args(ws, M, K, image, nullptr, nullptr, N, acc, fp6, plan);
    if (test_flags & CONVROT_TEST_SPLIT_TIMEOUT) {
        a.extra_wait = 1;  // one writer more than exist: every finalizer's wait runs out
        a.spin_limit = 64;
    }
    return enqueue_gemm(GEMM_OUT_I32, a, s);
}

}  // extern "C"
