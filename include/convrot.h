/*
 * convrot.h -- C ABI of the ConvRot W4A4 rotated linear for AMD Instinct
 * MI355X (gfx950).
 *
 * The operation (convrot-mlx README, "What is included"; comfy-quants issue
 * "convrot is ... QuaRot Stage 1c", section 1):
 *   Y[M,N] = bf16( (Q(X R) . Q(W R)^T) * sx[m] * sw[n] + bias[n] )
 * where R = I_G (x) H_g / sqrt(g) is the block-diagonal normalized Hadamard
 * rotation over contiguous groups of g in {64, 256} input channels -- H_g the
 * Sylvester matrix, or the regular one when g carries
 * CONVROT_REGULAR_HADAMARD (below) -- and Q quantizes each rotated row symmetrically to signed 4-bit codes in
 * [-7, 7] with one scale s = absmax(row) / 7 per row (codes rint(r / s),
 * ties to even; an all-zero row has s = 0 and codes 0).  The product is an
 * exact integer dot product; the epilogue is fmaf(float(acc) * sx[m], sw[n],
 * bias[n]) rounded to bf16 (nearest even).
 *
 * Conventions for every entry point:
 *   - Matrices are dense row-major; X is [M][K] and W is [N][K] (a weight row
 *     is an output channel), Y is [M][N].  bf16 tensors are passed as raw
 *     16-bit storage.
 *   - Pointers named *_dev are device pointers; pointers named *_host are host
 *     pointers.  The library never allocates, frees or retains device memory
 *     and keeps no state between calls: the caller owns every buffer (the one
 *     exception is the fixed device workspace of convrot_linear_noalloc,
 *     below, which lives as long as the process).
 *   - stream is a hipStream_t passed as void* (NULL = the null stream).  Device
 *     entry points only enqueue work on it and return; nothing is synchronised.
 *   - Device buffers must be 16-byte aligned except sw/sx/bias (4/4/2 bytes).
 *   - Sizes: K % 8 == 0 and K_rot <= 16384, where K_rot = K rounded up to a
 *     multiple of g; 0 <= M, N <= 16777216.  M == 0 or N == 0 is a no-op that
 *     returns CONVROT_OK.
 *   - When g does not divide K, every row of X and W is zero-padded to K_rot
 *     before the rotation (comfy-quants issue, section 1, which pads the last
 *     block when needed), and codes, scales and the product cover the K_rot rotated
 *     values; the result is still X W^T up to quantization.  Outputs that are
 *     rows of codes or rotated values are K_rot wide; X and W stay K wide.
 *   - All arguments are checked before anything is launched; on any error
 *     nothing is enqueued and an error status is returned.  There is no
 *     fallback path of any kind.
 *   - Calls on different streams may run concurrently; calls sharing a
 *     workspace must be ordered by the caller.
 */
#ifndef CONVROT_H
#define CONVROT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define CONVROT_OK 0
#define CONVROT_EINVAL 1     /* bad size, group, null or misaligned pointer   */
#define CONVROT_EWORKSPACE 2 /* workspace smaller than convrot_workspace_bytes */
#define CONVROT_EHIP 3       /* the HIP runtime reported an error at launch   */
#define CONVROT_EDEVICE 4    /* current device is not a gfx950 GPU            */

/* Human-readable text for a status code (static storage, never NULL). */
const char* convrot_status_string(int status);

/* Library version string, e.g. "convrot-gfx950 1.1". */
const char* convrot_version(void);

/* Rotation flag for every g argument: g = 64 or 256 selects the normalized
 * Sylvester matrix H_g / sqrt(g); g = (64 or 256) | CONVROT_REGULAR_HADAMARD
 * selects the normalized regular Hadamard matrix (J_4 - 2 I_4)^(x k) / sqrt(g),
 * g = 4^k, whose rows all sum to sqrt(g) (convrot-mlx README, "What is
 * included": normalized regular-Hadamard rotation; comfy-quants issue,
 * section 2: for 4^k it equals the Sylvester matrix up to signed permutations
 * of rows and columns).  A weight image is valid only with the g it was
 * prepared with: convrot_linear must be given the same value. */
#define CONVROT_REGULAR_HADAMARD 0x10000

/* Image flag for every g argument: the weight image holds the packed INT4
 * codes only, 0.5 bytes per weight -- the memory saving the pages aim at
 * (convrot-mlx README, "Why this repository exists") -- and every product
 * runs on the INT8 matrix cores.  Without it the image also carries the same
 * codes as FP6 e2m3 values (1.25 bytes per weight in all), which lets the
 * large-M product run on the FP6 matrix cores at twice the INT8 rate.  The
 * flag changes the sizes below and must be passed, like the rotation flag,
 * with the same value to every call that uses the image. */
#define CONVROT_INT4_IMAGE 0x20000

/* ---- sizes (host only, no HIP call) ----------------------------------- */

/* Bytes of the weight image for an N x K weight: the packed INT4 codes,
 * round_up(N, 32) * round_up(K_rot, 128) / 2 bytes in 32-column x 128-K
 * units in MFMA fragment order (convrot-mlx README, "What is included": the
 * K x packed-N family of layouts, here tiled for CDNA4 matrix cores), followed
 * -- unless g carries CONVROT_INT4_IMAGE -- by the same codes as FP6 e2m3
 * values (every integer in [-7, 7] is exact in e2m3), round_up(N, 32) *
 * round_up(K_rot, 128) * 3 / 4 bytes, for the FP6 matrix cores of the
 * large-M product.  g must be 64 or 256 (with or without the flags above).
 * Returns CONVROT_OK or CONVROT_EINVAL. */
int convrot_weight_image_bytes(int64_t N, int64_t K, int g, size_t* bytes_host);

/* Bytes of workspace convrot_linear needs for an M x K input and N outputs.
 * Layout, each part starting at a 256-byte boundary:
 *   1. offset 0: 512 uint32 counters of the split-K GEMM (cleared by the
 *      activation step, left cleared by every GEMM; at the same offset for
 *      every shape);
 *   2. offset CONVROT_WORKSPACE_STATUS_OFFSET: a uint32 status word, cleared
 *      by the activation step of every call (convrot_linear,
 *      convrot_prepare_activations, convrot_gemm_i32) and set to
 *      CONVROT_STATUS_SPLIT_TIMEOUT by a split-K GEMM whose last workgroup of
 *      a tile stopped waiting for the others' partial sums (a bounded wait of
 *      seconds; it then adds none of them, so that call's Y is wrong).  The
 *      library never reads it: a caller that wants to know reads the word
 *      after the call has completed;
 *   3. offset CONVROT_WORKSPACE_IMAGE_OFFSET: the activation-code image,
 *      round_up(M, 32) * round_up(K_rot, 128) / 2 bytes, INT4 codes in the
 *      same layout as the weight image;
 *   4. when M > 32 and g does not carry CONVROT_INT4_IMAGE, room for the same
 *      codes as FP6: round_up(M, 32) * round_up(K_rot, 128) * 3 / 4 bytes
 *      (convrot_prepare_activations writes both copies; convrot_linear
 *      writes only the one its plan reads: the FP6 copy when the plan runs on
 *      the FP6 matrix cores, the INT4 image otherwise);
 *   5. the activation scales sx: round_up(M, 32) floats;
 *   6. split-K partial tiles: when M > 128 and the output tiles are too few
 *      to occupy the GPU, each tile's K range is shared by S workgroups and
 *      S - 1 partial tiles of 4-byte sums per output tile live here (0 bytes
 *      otherwise).
 * Parts 1-5 depend on M, K and g only; convrot_prepare_activations needs only
 * them.  Returns CONVROT_OK or CONVROT_EINVAL. */
#define CONVROT_WORKSPACE_STATUS_OFFSET 2048
#define CONVROT_WORKSPACE_IMAGE_OFFSET 4096
#define CONVROT_STATUS_SPLIT_TIMEOUT 1
int convrot_workspace_bytes(int64_t M, int64_t K, int64_t N, int g, size_t* bytes_host);

/* *count = the number of kernels convrot_linear launches for this shape: 1
 * (M <= 4 with 1024 <= K <= 4096 for g = 256 or 512 <= K <= 2048 for g = 64),
 * 2 (activation kernel, then GEMM), or 0 (M or N is 0).  Returns CONVROT_OK
 * or CONVROT_EINVAL. */
int convrot_linear_kernel_count(int64_t M, int64_t K, int64_t N, int g, int* count_host);

/* The plan of convrot_linear's integer product for this shape, into host
 * ints: *mfma_kind = the matrix cores it runs on, CONVROT_MFMA_I8 (INT8 MFMA
 * on codes widened from INT4) or CONVROT_MFMA_FP6 (FP6 e2m3 MFMA on the FP6
 * copy of the codes; exact: the codes are exact e2m3 values and the binary32
 * sums are exact integers), 0 when M or N is 0; *tile_m x *tile_n = the block
 * tile when M > 128 (0 x 0 for the weight-streaming kernel of M <= 128);
 * *splits = workgroups sharing each tile's K range (1 when not split).
 * Returns CONVROT_OK or CONVROT_EINVAL. */
#define CONVROT_MFMA_I8 1
#define CONVROT_MFMA_FP6 2
int convrot_linear_plan(int64_t M, int64_t K, int64_t N, int g, int* mfma_kind_host, int* tile_m_host,
                        int* tile_n_host, int* splits_host);

/* ---- argument checks (host only, no HIP call) ------------------------- */

/* The checks convrot_prepare_weight performs.  Returns a status code. */
int convrot_validate_weight(const void* W_dev, int64_t N, int64_t K, int g, const void* image_dev,
                            const float* sw_dev);

/* The checks convrot_linear performs.  Returns a status code. */
int convrot_validate_linear(const void* X_dev, int64_t M, int64_t K, const void* image_dev,
                            const float* sw_dev, const void* bias_dev, int64_t N, int g, const void* Y_dev,
                            const void* workspace_dev, size_t ws_bytes);

/* ---- offline weight preparation --------------------------------------- */

/* Rotate every weight row by I_G (x) H_g / sqrt(g), quantize it rowwise to
 * INT4 codes in [-7, 7] with scale sw[n] = absmax / 7, and write the codes as
 * the packed weight image (convrot-mlx README, "Install and test": the
 * weight conversion step quantize_convrot_weight followed by the repack for
 * the matrix-core layout).
 *   W_dev     bf16 [N][K], read only.
 *   image_dev convrot_weight_image_bytes(N, K, g) bytes, fully written
 *             (padding included).  Valid only for this (N, K); the caller keeps
 *             g beside it and passes the same g to convrot_linear.
 *   sw_dev    float [N], written.
 */
int convrot_prepare_weight(const void* W_dev, int64_t N, int64_t K, int g, void* image_dev, float* sw_dev,
                           void* stream);

/* The same rotation and quantization, writing the portable N x packed-K form
 * (convrot-mlx README, "What is included": reversible N x packed-K layout):
 * qweight_nk_dev is uint8 [N][K_rot/2], byte j of row n holding code 2j in its low
 * nibble and code 2j+1 in its high nibble (two's complement).  sw_dev float [N]. */
int convrot_quantize_weight(const void* W_dev, int64_t N, int64_t K, int g, uint8_t* qweight_nk_dev,
                            float* sw_dev, void* stream);

/* Lossless repack of N x packed-K codes into the weight image (the analogue
 * of the pages' repack_nk_weight_for_mpp, convrot-mlx README, "Install and
 * test").  qweight_nk_dev is uint8 [N][K_rot/2]; image_dev:
 * convrot_weight_image_bytes(N, K, g) bytes (g only decides K_rot and whether
 * the FP6 copy is written). */
int convrot_repack_nk_to_image(const uint8_t* qweight_nk_dev, int64_t N, int64_t K, int g, void* image_dev,
                               void* stream);

/* ---- the linear ------------------------------------------------------- */

/* Y = the ConvRot W4A4 linear of X with a prepared weight (convrot-mlx
 * README, "Install and test": the complete path is rotation, activation
 * quantization, integer product, scaling and bias).
 *   X_dev      bf16 [M][K].
 *   image_dev  from convrot_prepare_weight / convrot_repack_nk_to_image with
 *              the same N, K (and g for prepare_weight).
 *   sw_dev     float [N].
 *   bias_dev   bf16 [N], or NULL for no bias.
 *   Y_dev      bf16 [M][N], written.
 *   workspace_dev / ws_bytes: at least convrot_workspace_bytes(M, K, N, g);
 *              its contents on entry are ignored and on exit hold the
 *              activation codes and scales of X: the codes in the copy the
 *              product reads -- the FP6 copy when convrot_linear_plan reports
 *              CONVROT_MFMA_FP6, the INT4 image otherwise.
 * For M <= 4 with 1024 <= K <= 4096 (g = 256) or 512 <= K <= 2048 (g = 64)
 * the whole linear is one kernel: every workgroup quantizes the few
 * activation rows itself, in shared memory, while its weight loads are in
 * flight; otherwise an activation kernel is followed by the GEMM.
 */
int convrot_linear(const void* X_dev, int64_t M, int64_t K, const void* image_dev, const float* sw_dev,
                   const void* bias_dev, int64_t N, int g, void* Y_dev, void* workspace_dev, size_t ws_bytes,
                   void* stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation: the same
 * linear as convrot_linear (same arguments and checks, same kernels, same
 * result bit for bit) with no workspace argument.  Its workspace is a
 * library-owned device array of CONVROT_NOALLOC_MAX_WORKSPACE bytes, one per
 * GPU, held until the process ends; the call allocates nothing (no hipMalloc,
 * no allocating library routine).  Shapes whose convrot_workspace_bytes(M, K,
 * N, g) exceeds that size return CONVROT_EWORKSPACE (every FLUX-shaped linear
 * fits).  All calls on one GPU share the array: calls that may overlap on one
 * GPU (different streams, or different host threads without ordering) race
 * and must be serialized by the caller.  The array keeps the last call's
 * contents; the parts that must start at zero (split-K counters, status
 * word) are cleared by a kernel of every call, so the call can be captured
 * in a HIP graph.  CONVROT_EHIP if the array's address cannot be found. */
#define CONVROT_NOALLOC_MAX_WORKSPACE (48u << 20)
int convrot_linear_noalloc(const void* X_dev, int64_t M, int64_t K, const void* image_dev, const float* sw_dev,
                           const void* bias_dev, int64_t N, int g, void* Y_dev, void* stream);

/* ---- W4A16 variant (weight-only INT4) ------------------------------------ */
/* The weight-bandwidth-bound regime, M <= 32 (convrot-mlx README, "What is
 * included": a W4A16 path beside W4A4).  The activation rows are rotated as
 * in convrot_linear and rounded to bf16 (nearest even) instead of being
 * quantized; the product runs against the same weight image:
 *   Y[m][n] = bf16( fmaf(sum_k bf16(r[m][k]) * qw[n][k], sw[n], bias[n]) ),
 * the sum accumulated in binary32 by the bf16 matrix cores (so Y is close to,
 * not bit-identical with, the same formula summed exactly).
 * Bytes of workspace for M x K: round_up(M, 16) * round_up(K_rot, 128) * 2.
 * It receives the bf16 rotated rows in the order the matrix cores read them:
 * value k of row m (kl = k % 128, b_i = bit i of kl, KB = round_up(K_rot,
 * 128) / 128) is element kl % 8 of the 16-byte word number
 *   ((((m / 16) * KB + k / 128) * 4 + 2 b5 + b3) * 4 + 2 b6 + b4) * 16 + m % 16;
 * the words of padding rows and columns are not written.  M must be <= 32;
 * otherwise, and for the shape rules of convrot_linear, CONVROT_EINVAL. */
int convrot_w4a16_workspace_bytes(int64_t M, int64_t K, int g, size_t* bytes_host);

/* The checks convrot_linear_w4a16 performs.  Returns a status code. */
int convrot_validate_linear_w4a16(const void* X_dev, int64_t M, int64_t K, const void* image_dev,
                                  const float* sw_dev, const void* bias_dev, int64_t N, int g, const void* Y_dev,
                                  const void* workspace_dev, size_t ws_bytes);

/* The W4A16 linear: arguments as convrot_linear (image_dev and sw_dev from
 * convrot_prepare_weight with the same g), workspace of at least
 * convrot_w4a16_workspace_bytes(M, K, g).  Two kernels on the stream. */
int convrot_linear_w4a16(const void* X_dev, int64_t M, int64_t K, const void* image_dev, const float* sw_dev,
                         const void* bias_dev, int64_t N, int g, void* Y_dev, void* workspace_dev, size_t ws_bytes,
                         void* stream);

/* The two halves of convrot_linear, for callers that want to time or reuse
 * them separately.  convrot_prepare_activations writes the activation codes
 * and scales of X into the workspace (rotation, row absmax, quantization);
 * convrot_gemm consumes that workspace: integer products against the weight
 * image, then the scale + bias epilogue into Y.  Same arguments and rules as
 * convrot_linear, except that convrot_prepare_activations needs only the
 * first five parts of the workspace (it does not know N).  convrot_gemm takes
 * the M, K, N and g of the linear.  It leaves the workspace valid for another
 * convrot_gemm. */
int convrot_prepare_activations(const void* X_dev, int64_t M, int64_t K, int g, void* workspace_dev,
                                size_t ws_bytes, void* stream);
int convrot_gemm(const void* workspace_dev, size_t ws_bytes, int64_t M, int64_t K, const void* image_dev,
                 const float* sw_dev, const void* bias_dev, int64_t N, int g, void* Y_dev, void* stream);

/* ---- parity hooks (same kernels, exposed intermediate results) ---------- */

/* Rotation + row absmax + quantization of `rows` bf16 rows, with plain
 * row-major outputs: codes_dev int8 [rows][K_rot], scales_dev float [rows], and,
 * if rotated_dev is not NULL, the rotated rows as float [rows][K_rot] (convrot-mlx
 * README, "What is included": the rotation and the rowwise quantizer). */
int convrot_prepare_rows(const void* X_dev, int64_t rows, int64_t K, int g, int8_t* codes_dev, float* scales_dev,
                         float* rotated_dev, void* stream);

/* The integer product alone: acc_dev int32 [M][N] = qx . codes(image)^T for
 * activation codes qx_dev int8 [M][K] (values in [-7, 7]; K the code width).
 * The codes are first re-laid-out into the workspace
 * (convrot_workspace_bytes(M, K, N, 64) bytes), then the GEMM kernel of
 * convrot_linear runs with its epilogue replaced by an int32 store.  The
 * image must carry its FP6 copy (prepared without CONVROT_INT4_IMAGE). */
int convrot_gemm_i32(const int8_t* qx_dev, int64_t M, int64_t K, const void* image_dev, int64_t N,
                     int32_t* acc_dev, void* workspace_dev, size_t ws_bytes, void* stream);

/* The same with the block-tile plan given instead of the library's choice
 * (M > 32): tile_m x tile_n one of 192 x 384 and 192 x 192 (INT8 matrix
 * cores, INT4 image part), 256 x 256 or 192 x (384 | CONVROT_TILE_FP6) (FP6
 * matrix cores, FP6 image part), and `splits` workgroups sharing each tile's
 * K range (1 .. min(8, K_pad / 128); a split launch may have at most 256
 * tiles x splits).  Lets a test reach every
 * block tile, with and without the split-K exchange, at any shape.  The
 * workspace must hold convrot_workspace_bytes_tiled(M, K, N, tile_m, tile_n,
 * splits) bytes -- sized from the same plan, so the exchange's partial tiles
 * fit.  test_flags: 0, or CONVROT_TEST_SPLIT_TIMEOUT to make the last
 * workgroup of every split tile wait for one writer more than exist, with a
 * tiny bound on the wait (it runs out, sets the status word and still ends
 * normally; the test of that report).  CONVROT_EINVAL for any other value. */
#define CONVROT_TEST_SPLIT_TIMEOUT 1
#define CONVROT_TILE_FP6 0x10000 /* or-ed into tile_n: the FP6 tile where both kinds have that size */
int convrot_workspace_bytes_tiled(int64_t M, int64_t K, int64_t N, int tile_m, int tile_n, int splits,
                                  size_t* bytes_host);
int convrot_gemm_i32_tiled(const int8_t* qx_dev, int64_t M, int64_t K, const void* image_dev, int64_t N,
                           int32_t* acc_dev, int tile_m, int tile_n, int splits, int test_flags, void* workspace_dev,
                           size_t ws_bytes, void* stream);

/* Host-side check of the split-K exchange of such a plan (no HIP call): every
 * byte offset the exchange stores to or copies from in the workspace's
 * partial-tile area, every counter slot and every LDS offset of the
 * finalizer's copies and reads, computed with the kernels' own address
 * functions; returns one past the largest of each: *partial_end_host (bytes
 * from the start of the partial area; to be <= the bytes that
 * convrot_workspace_bytes_tiled sets aside), *counters_used_host (counter
 * words; <= 512) and *lds_end_host (bytes of the stage ring).  All 0 when
 * splits == 1. */
int convrot_split_k_extent(int64_t M, int64_t K, int64_t N, int tile_m, int tile_n, int splits,
                           size_t* partial_end_host, int* counters_used_host, size_t* lds_end_host);

/* ---- measurement hook ---------------------------------------------------- */
/* The rate the matrix cores sustain on an MFMA-only loop -- operands in
 * registers, no memory traffic, two waves per SIMD as in the block tiles --
 * the practical denominator beside the published dense peak (under sustained
 * matrix-core load the clock stays below the peak figure's 2.4 GHz).  kind:
 * CONVROT_PROBE_FP6 (32x32x64 MFMA on FP6 e2m3 operands, 131072 ops each) or
 * CONVROT_PROBE_INT8 (32x32x32 INT8, 65536 ops each).  Each wave runs
 * `iterations` (1 .. 2^24) rounds of four independent MFMAs; out_dev receives
 * one float per thread (a checksum; its value carries no meaning) and must
 * hold *bytes from convrot_matrix_core_probe_bytes; *mfma_count_host = the
 * MFMA instructions the launch runs.  The caller times the launch on its
 * stream.  CONVROT_EINVAL for a bad kind, count or pointer, CONVROT_EWORKSPACE
 * for a short buffer. */
#define CONVROT_PROBE_FP6 1
#define CONVROT_PROBE_INT8 2
int convrot_matrix_core_probe_bytes(size_t* bytes_host);
int convrot_matrix_core_probe(int kind, int iterations, float* out_dev, size_t out_bytes, int64_t* mfma_count_host,
                              void* stream);

/* ---- host layout tools (host memory, no HIP call) ----------------------- */

/* int8 codes [N][K] <-> N x packed-K uint8 [N][K/2] (low nibble = even k). */
int convrot_host_pack_nk(const int8_t* codes_host, int64_t N, int64_t K, uint8_t* nk_host);
int convrot_host_unpack_nk(const uint8_t* nk_host, int64_t N, int64_t K, int8_t* codes_host);
/* N x packed-K [N][K/2] <-> K x packed-N [K][N/2] (low nibble = even n);
 * N and K even. */
int convrot_host_nk_to_kn(const uint8_t* nk_host, int64_t N, int64_t K, uint8_t* kn_host);
int convrot_host_kn_to_nk(const uint8_t* kn_host, int64_t N, int64_t K, uint8_t* nk_host);
/* N x packed-K <-> weight image (convrot_weight_image_bytes(N, K, 64) bytes);
 * image_to_nk ignores the padding. */
int convrot_host_nk_to_image(const uint8_t* nk_host, int64_t N, int64_t K, uint8_t* image_host);
int convrot_host_image_to_nk(const uint8_t* image_host, int64_t N, int64_t K, uint8_t* nk_host);
/* Activation-code image (workspace + CONVROT_WORKSPACE_IMAGE_OFFSET) -> int8
 * codes [M][K]. */
int convrot_host_act_image_to_codes(const uint8_t* image_host, int64_t M, int64_t K, int8_t* codes_host);
/* The FP6 copies, decoded: the FP6 part of a weight image -> N x packed-K,
 * and the FP6 activation image of a workspace (whole workspace, M > 32) ->
 * int8 codes [M][K].  K is the code width, a multiple of 64.  CONVROT_EINVAL
 * also when a field is not the e2m3 pattern of an integer in [-7, 7]. */
int convrot_host_image_fp6_to_nk(const uint8_t* image_host, int64_t N, int64_t K, uint8_t* nk_host);
int convrot_host_workspace_fp6_codes(const uint8_t* workspace_host, int64_t M, int64_t K, int8_t* codes_host);

#ifdef __cplusplus
}
#endif
#endif /* CONVROT_H */
