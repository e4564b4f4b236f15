// kernels.h -- launch interface between the C ABI and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convrot {

enum PrepOut { OUT_IMAGE = 0, OUT_ROWMAJOR = 2, OUT_NK = 3, OUT_LDS = 4, OUT_ROTATED_BF16 = 5 };
enum GemmOut { GEMM_OUT_BF16 = 0, GEMM_OUT_I32 = 1 };

struct PrepArgs {
    const uint16_t* X;   // bf16 [rows][K]
    int64_t rows;        // rows holding data
    int64_t rows_pad;    // rows written (image mode: rows rounded up to 32)
    int64_t K, K_pad;    // K: rotated row length (a whole number of groups); K_pad: K rounded up to 128 (image mode)
    int64_t ld;          // elements per row of X (<= K: the rest of a row is zero padding)
    uint8_t* out;        // codes in the layout of the mode (OUT_IMAGE: the INT4 image, or nullptr)
    uint8_t* out6;       // OUT_IMAGE only: the FP6 image of the same codes, or nullptr (not both null)
    float* scales;       // [rows]
    float* rotated;      // OUT_ROWMAJOR only: fp32 [rows][K] or nullptr
    uint32_t* zero;      // words cleared by workgroup 0 (split-K counters) or nullptr
    int zero_count;
    int team;            // lanes per row (set by launch_prep)
    int x_stream;        // team kernel: read X with non-temporal loads (keeps it out of the caches)
};

struct GemmArgs {
    const uint8_t* act;  // INT4 operand image of the activation codes
    const uint8_t* wgt;  // INT4 operand image of the weight codes
    const uint8_t* act6; // FP6 images of the same codes (block-tile FP6 shape)
    const uint8_t* wgt6;
    const float* sx;     // [M]
    const float* sw;     // [N]
    const uint16_t* bias;  // bf16 [N] or nullptr
    void* out;           // bf16 or int32 [M][N]
    int64_t M, N;
    int64_t K;           // reduction length (the W4A16 activation rows are K long)
    int MT, NT, KB;      // 32-row tiles, 32-column tiles, 128-K blocks
    int shape;           // block tile shape, tiles and K splits (gemm_plan)
    int tiles_m, tiles_n;
    int splits;
    uint32_t* counters;  // 2 * kSplitCounters zeroed words (tickets, then finished writers)
    int32_t* partial;    // (splits - 1) partial tiles per tile (int32 or binary32 sums)
    uint32_t* status;    // the workspace's status word (set on a split-K wait that ran out)
    int spin_limit;      // sleeps a split-K finalizer waits at most
    int extra_wait;      // test hook: writers the finalizer waits for beyond those that exist (normally 0)
};

// g: group size, optionally with the flags of layout.h (kRegularHadamard: the rotation matrix)
void launch_prep(int g, int mode, PrepArgs a, hipStream_t s);
void launch_gemm(int out_mode, GemmArgs a, hipStream_t s);
// W4A16 product for M <= 32: bf16 rotated activation rows xr [M][K] times the
// weight image (act, sx and the split fields of a are unused).
void launch_w4a16(GemmArgs a, const uint16_t* xr, hipStream_t s);
// The W4A16 linear in one launch when single_kernel_linear(M, K, g) holds:
// p.out receives the bf16 rotated rows [M][K].
void launch_small_w4a16(int g, GemmArgs a, PrepArgs p, hipStream_t s);
// Whole linear in one launch when single_kernel_linear(M, K, g) holds; see
// kernels.hip.
void launch_small_m(int g, GemmArgs a, PrepArgs p, hipStream_t s);
// Layout moves into the INT4 image and, when image6 is not null, the FP6 image.
void launch_act_relayout(const int8_t* codes, int64_t M, int64_t K, uint8_t* image, uint8_t* image6, uint32_t* zero,
                         int zero_count, hipStream_t s);
void launch_repack_nk(const uint8_t* nk, int64_t N, int64_t K, uint8_t* image, uint8_t* image6, hipStream_t s);

// Matrix-core rate probe: kind kProbeFp6 (32x32x64 FP6 e2m3) or kProbeInt8
// (32x32x32 INT8); probe_grid() workgroups of kProbeThreads threads, each
// wave running iters x 4 MFMAs; out holds one float per thread.
constexpr int kProbeFp6 = 1, kProbeInt8 = 2, kProbeThreads = 256;
int64_t probe_grid();
void launch_mfma_probe(int kind, int iters, float* out, hipStream_t s);

}  // namespace convrot
