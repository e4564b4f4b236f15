// host.cpp -- size queries, argument checks and host layout tools of the
// ConvRot C ABI.  Pure C++: nothing here calls the HIP runtime, so every
// function works on a machine without a GPU.
#include <string.h>

#include "../../include/convrot.h"
#include "internal.h"
#include "layout.h"

using namespace convrot;

static_assert(CONVROT_REGULAR_HADAMARD == kRegularHadamard, "header and library agree on the rotation flag");
static_assert(CONVROT_INT4_IMAGE == kInt4Image, "header and library agree on the image flag");
static_assert(CONVROT_STATUS_SPLIT_TIMEOUT == (int)kStatusSplitTimeout, "header and library agree on the status");
static_assert(CONVROT_WORKSPACE_STATUS_OFFSET == 4 * 2 * kSplitCounters, "status word right after the counters");
static_assert(CONVROT_TILE_FP6 == kTileFp6, "tile flag of the test hooks");
static_assert(CONVROT_WORKSPACE_IMAGE_OFFSET >= CONVROT_WORKSPACE_STATUS_OFFSET + 4 &&
                  CONVROT_WORKSPACE_IMAGE_OFFSET % 256 == 0,
              "activation image after the status word");

namespace convrot {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_shape(int64_t rows, int64_t K, int g)
{
    if ((g & ~kGroupFlags) != 64 && (g & ~kGroupFlags) != 256) return CONVROT_EINVAL;
    // rows of X and W are 16-byte aligned runs of bf16; the rotated width
    // (K rounded up to g, the rest zero padding) is at most kMaxK
    if (K < 1 || K % 8 != 0 || rotated_width(K, g) > kMaxK) return CONVROT_EINVAL;
    if (rows < 0 || rows > kMaxRows) return CONVROT_EINVAL;
    return CONVROT_OK;
}

// Workspace layout (each part 256-byte aligned): the split-K counters at
// offset 0 and the status word after them -- the same place for every shape,
// so a workspace reused across shapes keeps them cleared -- then the
// activation INT4 image, the activation FP6 image (M > 32, FP6 images), sx,
// and the split-K partial tiles.
size_t workspace_image_offset() { return CONVROT_WORKSPACE_IMAGE_OFFSET; }

size_t workspace_image6_offset(int64_t M, int64_t K)
{
    return (size_t)round_up((int64_t)(workspace_image_offset() + image_bytes(M, K)), 256);
}

size_t workspace_sx_offset(int64_t M, int64_t K, bool fp6)
{
    const size_t part6 = act_has_fp6(M, fp6) ? image6_bytes(M, K) : 0;
    return (size_t)round_up((int64_t)(workspace_image6_offset(M, K) + part6), 256);
}

size_t workspace_partial_offset(int64_t M, int64_t K, bool fp6)
{
    return (size_t)round_up((int64_t)(workspace_sx_offset(M, K, fp6) + sizeof(float) * (size_t)round_up(M, kTileRows)),
                            256);
}

size_t workspace_bytes_for(int64_t M, int64_t K, bool fp6, const GemmPlan& p)
{
    return workspace_partial_offset(M, K, fp6) + gemm_partial_bytes(p);
}

size_t workspace_bytes(int64_t M, int64_t K, int64_t N, bool fp6)
{
    return workspace_bytes_for(M, K, fp6, gemm_plan(M, N, K, fp6));
}

int check_forced_plan(int64_t M, int64_t K, int64_t N, int tile_m, int tile_n, int splits, bool fp6, GemmPlan* plan)
{
    const int shape = gemm_shape_of(tile_m, tile_n);
    if (shape < 0 || M <= 32 || N < 1 || K < 1) return CONVROT_EINVAL;
    if (gemm_shape_fp6(shape) && !fp6) return CONVROT_EINVAL;
    const int64_t KB = round_up(K, kTileK) / kTileK;
    if (splits < 1 || splits > kMaxSplits || splits > KB) return CONVROT_EINVAL;
    const GemmPlan p = gemm_plan_forced(M, N, shape, splits);
    if (splits > 1 && (int64_t)p.tiles_m * p.tiles_n * splits > kSplitCounters) return CONVROT_EINVAL;
    *plan = p;
    return CONVROT_OK;
}

}  // namespace convrot

extern "C" {

const char* convrot_status_string(int status)
{
    switch (status) {
        case CONVROT_OK: return "ok";
        case CONVROT_EINVAL: return "invalid argument (size, group, null or misaligned pointer)";
        case CONVROT_EWORKSPACE: return "workspace too small";
        case CONVROT_EHIP: return "HIP runtime error at launch";
        case CONVROT_EDEVICE: return "current device is not a gfx950 GPU";
        default: return "unknown status";
    }
}

const char* convrot_version(void) { return "convrot-gfx950 1.1"; }

int convrot_weight_image_bytes(int64_t N, int64_t K, int g, size_t* bytes)
{
    if (!bytes) return CONVROT_EINVAL;
    int rc = check_shape(N, K, g);
    if (rc) return rc;
    *bytes = weight_image_bytes(N, rotated_width(K, g), image_has_fp6(g));
    return CONVROT_OK;
}

int convrot_workspace_bytes(int64_t M, int64_t K, int64_t N, int g, size_t* bytes)
{
    if (!bytes) return CONVROT_EINVAL;
    int rc = check_shape(M, K, g);
    if (rc) return rc;
    if (N < 0 || N > kMaxRows) return CONVROT_EINVAL;
    *bytes = workspace_bytes(M, rotated_width(K, g), N, image_has_fp6(g));
    return CONVROT_OK;
}

int convrot_workspace_bytes_tiled(int64_t M, int64_t K, int64_t N, int tile_m, int tile_n, int splits, size_t* bytes)
{
    if (!bytes) return CONVROT_EINVAL;
    int rc = check_shape(M, K, 64);
    if (rc) return rc;
    if (N < 0 || N > kMaxRows) return CONVROT_EINVAL;
    GemmPlan p;
    const bool fp6 = gemm_shape_fp6(gemm_shape_of(tile_m, tile_n));
    if ((rc = check_forced_plan(M, K, N, tile_m, tile_n, splits, fp6, &p))) return rc;
    *bytes = workspace_bytes_for(M, K, fp6, p);
    return CONVROT_OK;
}

int convrot_split_k_extent(int64_t M, int64_t K, int64_t N, int tile_m, int tile_n, int splits, size_t* partial_end,
                           int* counters_used, size_t* lds_end)
{
    if (!partial_end || !counters_used || !lds_end) return CONVROT_EINVAL;
    int rc = check_shape(M, K, 64);
    if (rc) return rc;
    GemmPlan p;
    if ((rc = check_forced_plan(M, K, N, tile_m, tile_n, splits, true, &p))) return rc;
    const int shape = p.shape;
    const int tiles = p.tiles_m * p.tiles_n;
    const int threads = gemm_threads(shape), words = split_words_per_thread(shape);
    const int pairs = split_pairs(shape), chunks = split_pair_bytes(shape) / 1024;  // 1 KB copies per pair
    size_t pend = 0, lend = 0;
    int cmax = -1;
    if (splits > 1) {
        // every address the exchange touches, through the kernels' own geometry
        for (int tile = 0; tile < tiles; ++tile) {
            for (int sub = 0; sub < splits; ++sub) {
                // tickets and finished writers of sub-block `sub`
                const int c = split_counter(tile, splits, sub) + kSplitCounters;
                cmax = c > cmax ? c : cmax;
            }
            for (int ticket = 0; ticket < splits - 1; ++ticket)
                for (int u = 0; u < words; ++u)
                    for (int t = 0; t < threads; ++t) {
                        const size_t end = split_store_offset(shape, tile, splits, ticket, u, t) + 8;
                        pend = end > pend ? end : pend;
                    }
            // the finalizer's copies: pair pr of every slot, into ring position
            // (m mod split_pairs_per_copy) for the m-th pair of its sub-block
            for (int sl = 0; sl < splits - 1; ++sl)
                for (int pr = 0; pr < pairs; ++pr)
                    for (int c = 0; c < chunks; ++c)
                        for (int lane = 0; lane < 64; ++lane) {
                            const size_t end = split_copy_offset(shape, tile, splits, sl, pr, c, lane) + 16;
                            pend = end > pend ? end : pend;
                            const int i = pr % gemm_wave_tiles_m(shape), j = pr / gemm_wave_tiles_m(shape);
                            const int m = i * gemm_wave_tiles_n(shape) + j -
                                          split_sub_first(shape, splits, split_sub_of(shape, splits, i, j));
                            const size_t lds = (size_t)(m % split_pairs_per_copy(shape)) * split_pair_bytes(shape) +
                                               (size_t)c * 1024 + (size_t)lane * 16 + 16;
                            lend = lds > lend ? lds : lend;
                        }
        }
    }
    *partial_end = pend;
    *counters_used = cmax + 1;
    *lds_end = lend;
    return CONVROT_OK;
}

int convrot_linear_kernel_count(int64_t M, int64_t K, int64_t N, int g, int* count)
{
    if (!count) return CONVROT_EINVAL;
    int rc = check_shape(M, K, g);
    if (rc) return rc;
    if (N < 0 || N > kMaxRows) return CONVROT_EINVAL;
    *count = (M == 0 || N == 0) ? 0 : single_kernel_linear(M, rotated_width(K, g), g) ? 1 : 2;
    return CONVROT_OK;
}

int convrot_linear_plan(int64_t M, int64_t K, int64_t N, int g, int* kind, int* tile_m, int* tile_n, int* splits)
{
    if (!kind || !tile_m || !tile_n || !splits) return CONVROT_EINVAL;
    int rc = check_shape(M, K, g);
    if (rc) return rc;
    if (N < 0 || N > kMaxRows) return CONVROT_EINVAL;
    *kind = 0;
    *tile_m = *tile_n = 0;
    *splits = 1;
    if (M == 0 || N == 0) return CONVROT_OK;
    // M <= kStreamMaxRows streams the weight through the INT8 16x16x64 MFMA
    *kind = CONVROT_MFMA_I8;
    if (M <= kStreamMaxRows) return CONVROT_OK;
    const GemmPlan p = gemm_plan(M, N, rotated_width(K, g), image_has_fp6(g));
    if (gemm_shape_fp6(p.shape)) *kind = CONVROT_MFMA_FP6;
    *tile_m = gemm_tile_m(p.shape);
    *tile_n = gemm_tile_n(p.shape);
    *splits = p.splits;
    return CONVROT_OK;
}

int convrot_validate_weight(const void* W, int64_t N, int64_t K, int g, const void* image, const float* sw)
{
    int rc = check_shape(N, K, g);
    if (rc) return rc;
    if (N == 0) return CONVROT_OK;
    if (!W || !image || !sw) return CONVROT_EINVAL;
    if (!aligned(W, 16) || !aligned(image, 16) || !aligned(sw, 4)) return CONVROT_EINVAL;
    return CONVROT_OK;
}

int convrot_validate_linear(const void* X, int64_t M, int64_t K, const void* image, const float* sw,
                            const void* bias, int64_t N, int g, const void* Y, const void* ws, size_t ws_bytes)
{
    int rc = check_shape(M, K, g);
    if (rc) return rc;
    if (N < 0 || N > kMaxRows) return CONVROT_EINVAL;
    if (M == 0 || N == 0) return CONVROT_OK;
    if (!X || !image || !sw || !Y || !ws) return CONVROT_EINVAL;
    if (!aligned(X, 16) || !aligned(image, 16) || !aligned(Y, 16) || !aligned(ws, 16)) return CONVROT_EINVAL;
    if (!aligned(sw, 4) || (bias && !aligned(bias, 2))) return CONVROT_EINVAL;
    if (ws_bytes < workspace_bytes(M, rotated_width(K, g), N, image_has_fp6(g))) return CONVROT_EWORKSPACE;
    return CONVROT_OK;
}

int convrot_w4a16_workspace_bytes(int64_t M, int64_t K, int g, size_t* bytes)
{
    if (!bytes) return CONVROT_EINVAL;
    int rc = check_shape(M, K, g);
    if (rc) return rc;
    if (M > kW4A16MaxRows) return CONVROT_EINVAL;
    *bytes = w16_rows_bytes(M, rotated_width(K, g));
    return CONVROT_OK;
}

int convrot_validate_linear_w4a16(const void* X, int64_t M, int64_t K, const void* image, const float* sw,
                                  const void* bias, int64_t N, int g, const void* Y, const void* ws, size_t ws_bytes)
{
    size_t need = 0;
    int rc = convrot_w4a16_workspace_bytes(M, K, g, &need);
    if (rc) return rc;
    if (N < 0 || N > kMaxRows) return CONVROT_EINVAL;
    if (M == 0 || N == 0) return CONVROT_OK;
    if (!X || !image || !sw || !Y || !ws) return CONVROT_EINVAL;
    if (!aligned(X, 16) || !aligned(image, 16) || !aligned(Y, 16) || !aligned(ws, 16)) return CONVROT_EINVAL;
    if (!aligned(sw, 4) || (bias && !aligned(bias, 2))) return CONVROT_EINVAL;
    if (ws_bytes < need) return CONVROT_EWORKSPACE;
    return CONVROT_OK;
}

// ---- host layout tools ---------------------------------------------------

static inline uint8_t lo4(int8_t q) { return (uint8_t)q & 0x0F; }
static inline int8_t sext4(uint8_t v) { return (int8_t)((int8_t)(v << 4) >> 4); }

int convrot_host_pack_nk(const int8_t* codes, int64_t N, int64_t K, uint8_t* nk)
{
    if (!codes || !nk || N < 0 || K < 2 || K % 2) return CONVROT_EINVAL;
    for (int64_t n = 0; n < N; ++n) {
        const int8_t* q = codes + n * K;
        uint8_t* p = nk + n * (K / 2);
        for (int64_t j = 0; j < K / 2; ++j) p[j] = (uint8_t)(lo4(q[2 * j]) | (lo4(q[2 * j + 1]) << 4));
    }
    return CONVROT_OK;
}

int convrot_host_unpack_nk(const uint8_t* nk, int64_t N, int64_t K, int8_t* codes)
{
    if (!codes || !nk || N < 0 || K < 2 || K % 2) return CONVROT_EINVAL;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < K / 2; ++j) {
            uint8_t b = nk[n * (K / 2) + j];
            codes[n * K + 2 * j] = sext4(b & 0x0F);
            codes[n * K + 2 * j + 1] = sext4(b >> 4);
        }
    return CONVROT_OK;
}

// Nibble of code (n, k) in an N x packed-K buffer.
static inline uint8_t nk_nib(const uint8_t* nk, int64_t K, int64_t n, int64_t k)
{
    uint8_t b = nk[n * (K / 2) + k / 2];
    return (k & 1) ? (uint8_t)(b >> 4) : (uint8_t)(b & 0x0F);
}

int convrot_host_nk_to_kn(const uint8_t* nk, int64_t N, int64_t K, uint8_t* kn)
{
    if (!nk || !kn || N < 2 || K < 2 || N % 2 || K % 2) return CONVROT_EINVAL;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N / 2; ++j)
            kn[k * (N / 2) + j] = (uint8_t)(nk_nib(nk, K, 2 * j, k) | (nk_nib(nk, K, 2 * j + 1, k) << 4));
    return CONVROT_OK;
}

int convrot_host_kn_to_nk(const uint8_t* kn, int64_t N, int64_t K, uint8_t* nk)
{
    if (!nk || !kn || N < 2 || K < 2 || N % 2 || K % 2) return CONVROT_EINVAL;
    // K x packed-N is N x packed-K with the roles of N and K swapped
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < K / 2; ++j)
            nk[n * (K / 2) + j] = (uint8_t)(nk_nib(kn, N, 2 * j, n) | (nk_nib(kn, N, 2 * j + 1, n) << 4));
    return CONVROT_OK;
}

// Six-bit field of code (row, k) in an FP6 image: bit i of the field is bit
// 6 (k % 128) + i of the row's logical byte string.
static void fp6_put(uint8_t* image6, int64_t row, int64_t k, int64_t K_pad, uint32_t v)
{
    for (int i = 0; i < 6; ++i) {
        const int bit = 6 * (int)(k % kTileK) + i;
        uint8_t* p = image6 + image6_byte_offset(row, k / kTileK, bit >> 3, K_pad);
        *p = (uint8_t)((*p & ~(1u << (bit & 7))) | (((v >> i) & 1u) << (bit & 7)));
    }
}

static uint32_t fp6_get(const uint8_t* image6, int64_t row, int64_t k, int64_t K_pad)
{
    uint32_t v = 0;
    for (int i = 0; i < 6; ++i) {
        const int bit = 6 * (int)(k % kTileK) + i;
        v |= (uint32_t)((image6[image6_byte_offset(row, k / kTileK, bit >> 3, K_pad)] >> (bit & 7)) & 1u) << i;
    }
    return v;
}

// e2m3 bit pattern -> code in [-7, 7]; -128 for a pattern that is no such code
static int8_t fp6_code(uint32_t v)
{
    for (int q = -7; q <= 7; ++q)
        if (fp6_e2m3(q) == v) return (int8_t)q;
    return (int8_t)-128;
}

int convrot_host_nk_to_image(const uint8_t* nk, int64_t N, int64_t K, uint8_t* image)
{
    if (!nk || !image || N < 0 || K < 64 || K % 64 || K > kMaxK) return CONVROT_EINVAL;
    const int64_t K_pad = round_up(K, kTileK);
    memset(image, 0, weight_image_bytes(N, K, true));
    uint8_t* image6 = image + weight_image6_offset(N, K);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; k += 8) {
            uint32_t word = 0;
            for (int b = 0; b < 4; ++b)
                word |= (uint32_t)(nk_nib(nk, K, n, k + b) | (nk_nib(nk, K, n, k + 4 + b) << 4)) << (8 * b);
            memcpy(image + image_word_offset(n, k, K_pad), &word, 4);
            for (int e = 0; e < 8; ++e) fp6_put(image6, n, k + e, K_pad, fp6_e2m3(sext4(nk_nib(nk, K, n, k + e))));
        }
    return CONVROT_OK;
}

int convrot_host_image_fp6_to_nk(const uint8_t* image, int64_t N, int64_t K, uint8_t* nk)
{
    if (!nk || !image || N < 0 || K < 64 || K % 64 || K > kMaxK) return CONVROT_EINVAL;
    const int64_t K_pad = round_up(K, kTileK);
    const uint8_t* image6 = image + weight_image6_offset(N, K);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < K / 2; ++j) {
            const int8_t c0 = fp6_code(fp6_get(image6, n, 2 * j, K_pad));
            const int8_t c1 = fp6_code(fp6_get(image6, n, 2 * j + 1, K_pad));
            if (c0 == -128 || c1 == -128) return CONVROT_EINVAL;
            nk[n * (K / 2) + j] = (uint8_t)(((uint8_t)c0 & 0x0F) | (((uint8_t)c1 & 0x0F) << 4));
        }
    return CONVROT_OK;
}

int convrot_host_workspace_fp6_codes(const uint8_t* workspace, int64_t M, int64_t K, int8_t* codes)
{
    if (!workspace || !codes || M <= 32 || M > kMaxRows || K < 64 || K % 64 || K > kMaxK) return CONVROT_EINVAL;
    const int64_t K_pad = round_up(K, kTileK);
    const uint8_t* image6 = workspace + workspace_image6_offset(M, K);
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) {
            const int8_t c = fp6_code(fp6_get(image6, m, k, K_pad));
            if (c == -128) return CONVROT_EINVAL;
            codes[m * K + k] = c;
        }
    return CONVROT_OK;
}

int convrot_host_image_to_nk(const uint8_t* image, int64_t N, int64_t K, uint8_t* nk)
{
    if (!nk || !image || N < 0 || K < 64 || K % 64 || K > kMaxK) return CONVROT_EINVAL;
    const int64_t K_pad = round_up(K, kTileK);
    memset(nk, 0, (size_t)N * (size_t)(K / 2));
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; k += 8) {
            uint32_t word;
            memcpy(&word, image + image_word_offset(n, k, K_pad), 4);
            uint8_t* p = nk + n * (K / 2) + k / 2;
            for (int b = 0; b < 4; ++b) {
                uint8_t byte = (uint8_t)(word >> (8 * b));
                uint8_t c_lo = byte & 0x0F;   // code k + b
                uint8_t c_hi = byte >> 4;     // code k + 4 + b
                int e0 = b, e1 = 4 + b;       // positions within the 8 codes
                p[e0 / 2] |= (e0 & 1) ? (uint8_t)(c_lo << 4) : c_lo;
                p[e1 / 2] |= (e1 & 1) ? (uint8_t)(c_hi << 4) : c_hi;
            }
        }
    return CONVROT_OK;
}

int convrot_host_act_image_to_codes(const uint8_t* image, int64_t M, int64_t K, int8_t* codes)
{
    if (!image || !codes || M < 0 || K < 64 || K % 64 || K > kMaxK) return CONVROT_EINVAL;
    const int64_t K_pad = round_up(K, kTileK);
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; k += 8) {
            uint32_t word;
            memcpy(&word, image + image_word_offset(m, k, K_pad), 4);
            for (int b = 0; b < 4; ++b) {
                const uint8_t byte = (uint8_t)(word >> (8 * b));
                codes[m * K + k + b] = sext4(byte & 0x0F);
                codes[m * K + k + 4 + b] = sext4(byte >> 4);
            }
        }
    return CONVROT_OK;
}

}  // extern "C"
