/*
 * convrot_oracle.c -- plain, slow CPU definition of the ConvRot W4A4 linear.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product: it is
 * loaded by the test suite, by the package's smoke check and by the benchmark's
 * CPU-baseline leg, and by nothing else.  It shares no code, header, table or
 * helper with the HIP library, and the HIP library never calls it.
 *
 * Every function is the definition written out with plain loops, in the order
 * the pages state the method:
 *
 *   1. Split K into G = K/g contiguous groups, g in {64, 256}, and rotate each
 *      group of every row by the normalized Hadamard matrix H_g / sqrt(g); this
 *      is the block-diagonal operator R = I_G (x) H_g.
 *        [convrot-mlx README, "What is included": normalized Hadamard rotation
 *         for group sizes 64 and 256]
 *        [comfy-quants issue "convrot is ... QuaRot Stage 1c", section 1
 *         "Both apply group-wise operator": R = I_G (x) H_{N0} and
 *         X.R = [X_1 H, ..., X_G H]]
 *      H is the Sylvester matrix (recursive doubling), natural order; or,
 *      when the group-size argument carries ORACLE_REGULAR, the regular
 *      Hadamard matrix (J_4 - 2 I_4) (x) ... (x) (J_4 - 2 I_4), k factors for
 *      g = 4^k (every row sums to 2^k).
 *        [convrot-mlx README, "What is included": normalized regular-Hadamard
 *         rotation for group sizes 64 and 256]
 *        [comfy-quants issue, section 2 "The equivalent Hadamard matrix": for
 *         N0 = 4^k the regular and Sylvester matrices differ by signed
 *         permutations of rows and columns]
 *   2. Quantize every rotated row symmetrically to signed 4-bit codes in
 *      [-7, 7] with one absmax/7 scale per row.
 *        [convrot-mlx README, "What is included": symmetric signed W4/A4
 *         rowwise absmax quantization in [-7, 7]]
 *   3. Pack codes two per byte (N x packed-K) and the lossless transposed
 *      K x packed-N layout.
 *        [convrot-mlx README, "What is included": reversible N x packed-K and
 *         K x packed-N layouts]
 *   4. Integer dot products of activation codes with weight codes.
 *        [convrot-mlx README, "Requirements": signed INT8 x INT4 products]
 *   5. Rescale by the two row scales and add the bias, output bf16.
 *        [convrot-mlx README, "Install and test": the complete linear path is
 *         rotation, activation quantization, integer product, scaling, bias]
 *
 *   W4A16 variant (weight-only INT4): the activation rows are rotated as in
 *   step 1 and rounded to bf16 instead of being quantized, then multiplied by
 *   the same INT4 weight codes; y = fmaf(fl32(sum), sw[n], bias[n]) to bf16.
 *        [convrot-mlx README, "What is included": the W4A16 path beside W4A4]
 *
 * Row length: when K is not a multiple of g the rows are padded with zeros to
 * K_rot = round_up(K, g) before the rotation, and every later step works on
 * the K_rot rotated values (the padded X and W rows give the same X W^T).
 *        [comfy-quants issue, section 1: K = G N0, "or after padding the last
 *         block if necessary"]
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes):
 *   - rotation is computed in double as a dense g x g product per group and
 *     rounded once to binary32.  For bf16 inputs whose magnitudes within one
 *     group span fewer than ~37 binary orders the double sum is exact, so the
 *     binary32 value is the correctly rounded exact rotation.
 *   - scale s = fl32(a / 7) with a = max |r| over the whole row (binary32
 *     division, correctly rounded); an all-zero row has s = 0 and codes 0.
 *   - code q = clamp(rint(fl32(r / s)), -7, 7), round half to even.
 *   - nibbles are two's complement; the low nibble holds the even index.
 *   - epilogue y = fmaf(fl32(float(acc) * sx[m]), sw[n], bias[n]) and then
 *     bf16 round-to-nearest-even; the binary32 value y is exposed
 *     (oracle_epilogue_f32) so that its single rounding can be checked.
 *
 * Built with -O2 -ffp-contract=off so no multiply-add is fused behind the
 * source's back; the one fused multiply-add of the epilogue is an explicit
 * fmaf().
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* bf16 <-> binary32                                                          */
/* ------------------------------------------------------------------------ */

/* A bf16 value is the upper 16 bits of the binary32 with the same value. */
float oracle_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a finite binary32 to the nearest bf16, ties to the even bf16.
 * Written as "compare the distances to the two neighbouring bf16 values",
 * which is the definition of round-to-nearest-even. */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint16_t toward_zero = (uint16_t)(u >> 16);      /* |lo| <= |f|        */
    uint16_t away = (uint16_t)(toward_zero + 1);       /* next bf16 outward  */
    double d_lo = fabs((double)f - (double)oracle_bf16_to_f32(toward_zero));
    double d_hi = fabs((double)oracle_bf16_to_f32(away) - (double)f);
    if (d_lo < d_hi) return toward_zero;
    if (d_hi < d_lo) return away;
    return (toward_zero & 1u) ? away : toward_zero;   /* tie: even one      */
}

void oracle_f32_to_bf16_array(const float* f, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_bf16(f[i]);
}

/* ------------------------------------------------------------------------ */
/* Row-parallel helper: plain pthreads, each thread takes a contiguous slice  */
/* of rows.  The result never depends on the thread count.                    */
/* ------------------------------------------------------------------------ */

typedef void (*row_fn)(void* ctx, int64_t row);

struct slice {
    row_fn fn;
    void* ctx;
    int64_t begin, end;
};

static void* run_slice(void* p)
{
    struct slice* s = (struct slice*)p;
    for (int64_t r = s->begin; r < s->end; ++r) s->fn(s->ctx, r);
    return NULL;
}

static void parallel_rows(row_fn fn, void* ctx, int64_t rows, int nthreads)
{
    if (rows <= 0) return;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > rows) nthreads = (int)rows;
    pthread_t tid[256];
    int created[256];
    struct slice sl[256];
    int64_t per = (rows + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        created[t] = 0;
        sl[t].fn = fn;
        sl[t].ctx = ctx;
        sl[t].begin = (int64_t)t * per < rows ? (int64_t)t * per : rows;
        sl[t].end = sl[t].begin + per < rows ? sl[t].begin + per : rows;
    }
    /* slice 0 runs on the calling thread; a slice whose thread cannot be
     * started also runs on the calling thread */
    for (int t = 1; t < nthreads; ++t)
        if (sl[t].begin < sl[t].end && pthread_create(&tid[t], NULL, run_slice, &sl[t]) == 0) created[t] = 1;
    run_slice(&sl[0]);
    for (int t = 1; t < nthreads; ++t) {
        if (created[t])
            pthread_join(tid[t], NULL);
        else
            run_slice(&sl[t]);
    }
}

/* ------------------------------------------------------------------------ */
/* 1. Sylvester Hadamard matrix by recursive doubling:                        */
/*      H_1 = [1],  H_2n = [[H_n, H_n], [H_n, -H_n]].                        */
/* ------------------------------------------------------------------------ */

/* Returns 0 on success, -1 if g is not a power of two in [1, 4096]. */
int oracle_sylvester(int g, int8_t* H)
{
    if (g < 1 || g > 4096 || (g & (g - 1)) != 0) return -1;
    H[0] = 1;
    for (int n = 1; n < g; n *= 2) {
        for (int i = 0; i < n; ++i) {
            for (int j = 0; j < n; ++j) {
                int8_t v = H[(int64_t)i * g + j];
                H[(int64_t)i * g + (j + n)] = v;
                H[(int64_t)(i + n) * g + j] = v;
                H[(int64_t)(i + n) * g + (j + n)] = (int8_t)-v;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* 1b. Regular Hadamard matrix of order 4^k by Kronecker powers of the       */
/*     order-4 regular matrix B = J_4 - 2 I_4 (-1 on the diagonal, +1 off):  */
/*       R_4 = B,  R_4n = B (x) R_n  (block (a, b) is B[a][b] * R_n).        */
/* ------------------------------------------------------------------------ */

/* Group-size flag: rotate with the regular matrix instead of Sylvester. */
#define ORACLE_REGULAR 0x10000

/* Returns 0 on success, -1 if g is not a power of four in [4, 4096]. */
int oracle_regular_hadamard(int g, int8_t* H)
{
    if (g < 4 || g > 4096 || (g & (g - 1)) != 0) return -1;
    int k = 0;
    while ((1 << (2 * k)) < g) ++k;
    if ((1 << (2 * k)) != g) return -1;
    static const int8_t B[4][4] = {{-1, 1, 1, 1}, {1, -1, 1, 1}, {1, 1, -1, 1}, {1, 1, 1, -1}};
    /* build R_n for n = 4, 16, ... in the top-left corner of H */
    for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) H[(int64_t)i * g + j] = B[i][j];
    for (int n = 4; n < g; n *= 4) {
        /* R_4n = B (x) R_n; fill blocks (a, b) != (0, 0) first, then block (0, 0) */
        for (int a = 3; a >= 0; --a)
            for (int b = 3; b >= 0; --b)
                for (int i = 0; i < n; ++i)
                    for (int j = 0; j < n; ++j)
                        H[(int64_t)(a * n + i) * g + (b * n + j)] = (int8_t)(B[a][b] * H[(int64_t)i * g + j]);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* 2. Grouped rotation r = x (I_G (x) H_g) / sqrt(g), row vector times matrix */
/* ------------------------------------------------------------------------ */

struct rot_ctx {
    const uint16_t* X;
    int64_t K_in; /* elements per input row */
    int64_t K;    /* rotated row length: K_in rounded up to g */
    int g;
    const int8_t* H;
    double inv_norm; /* 1 / sqrt(g): 1/8 or 1/16, exact in double */
    float* R;
};

static void rotate_one_row(void* p, int64_t m)
{
    struct rot_ctx* c = (struct rot_ctx*)p;
    const uint16_t* x = c->X + m * c->K_in;
    float* r = c->R + m * c->K;
    const int g = c->g;
    for (int64_t base = 0; base < c->K; base += g) {
        for (int j = 0; j < g; ++j) {
            double acc = 0.0;
            for (int t = 0; t < g; ++t) {
                const double v = base + t < c->K_in ? (double)oracle_bf16_to_f32(x[base + t]) : 0.0; /* zero pad */
                acc += v * (double)c->H[(int64_t)t * g + j];
            }
            r[base + j] = (float)(acc * c->inv_norm); /* one rounding to binary32 */
        }
    }
}

/* Rotated row length for K input values and group argument g_arg. */
int64_t oracle_rotated_width(int64_t K, int g_arg)
{
    const int64_t g = g_arg & ~ORACLE_REGULAR;
    return g > 0 ? (K + g - 1) / g * g : K;
}

/* X: bf16 bits [rows][K]; R: binary32 [rows][K_rot], K_rot = K rounded up to
 * g.  g_arg is the group size, optionally with ORACLE_REGULAR.  Returns 0, or
 * -1 on bad arguments (g not a power of two -- of four for the regular
 * matrix). */
int oracle_rotate_rows(const uint16_t* X, int64_t rows, int64_t K, int g_arg, float* R, int nthreads)
{
    const int regular = (g_arg & ORACLE_REGULAR) != 0;
    const int g = g_arg & ~ORACLE_REGULAR;
    if (g < 2 || (g & (g - 1)) != 0 || g > 4096 || K <= 0 || rows < 0) return -1;
    int8_t* H = (int8_t*)malloc((size_t)g * g);
    if (!H) return -2;
    if ((regular ? oracle_regular_hadamard(g, H) : oracle_sylvester(g, H)) != 0) {
        free(H);
        return -1;
    }
    struct rot_ctx c = {X, K, oracle_rotated_width(K, g_arg), g, H, 1.0 / sqrt((double)g), R};
    parallel_rows(rotate_one_row, &c, rows, nthreads);
    free(H);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* 3. Symmetric rowwise absmax quantization to [-7, 7]                        */
/* ------------------------------------------------------------------------ */

struct q_ctx {
    const float* R;
    int64_t K;
    int8_t* Q;
    float* S;
};

static void quantize_one_row(void* p, int64_t m)
{
    struct q_ctx* c = (struct q_ctx*)p;
    const float* r = c->R + m * c->K;
    int8_t* q = c->Q + m * c->K;
    float a = 0.0f;
    for (int64_t k = 0; k < c->K; ++k) {
        float v = fabsf(r[k]);
        if (v > a) a = v;
    }
    if (a == 0.0f) {
        c->S[m] = 0.0f;
        for (int64_t k = 0; k < c->K; ++k) q[k] = 0;
        return;
    }
    float s = a / 7.0f; /* binary32 division, correctly rounded */
    c->S[m] = s;
    for (int64_t k = 0; k < c->K; ++k) {
        float t = rintf(r[k] / s); /* round half to even */
        if (t > 7.0f) t = 7.0f;
        if (t < -7.0f) t = -7.0f;
        q[k] = (int8_t)t;
    }
}

int oracle_quantize_rows(const float* R, int64_t rows, int64_t K, int8_t* Q, float* S, int nthreads)
{
    if (rows < 0 || K <= 0) return -1;
    struct q_ctx c = {R, K, Q, S};
    parallel_rows(quantize_one_row, &c, rows, nthreads);
    return 0;
}

/* Rotate + quantize: the whole per-row preparation (used for both the
 * activation rows X and the weight rows W).  X is [rows][K]; Q and R are
 * [rows][K_rot]. */
int oracle_prepare_rows(const uint16_t* X, int64_t rows, int64_t K, int g, int8_t* Q, float* S,
                        float* R_or_null, int nthreads)
{
    const int64_t Kr = oracle_rotated_width(K, g);
    float* R = R_or_null;
    if (!R) {
        R = (float*)malloc((size_t)(rows > 0 ? rows : 1) * (size_t)Kr * sizeof(float));
        if (!R) return -2;
    }
    int rc = oracle_rotate_rows(X, rows, K, g, R, nthreads);
    if (rc == 0) rc = oracle_quantize_rows(R, rows, Kr, Q, S, nthreads);
    if (!R_or_null) free(R);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* 4. Packing: two's complement nibbles, low nibble = even index              */
/* ------------------------------------------------------------------------ */

static uint8_t nibble(int8_t q) { return (uint8_t)((uint8_t)q & 0x0Fu); }

static int8_t from_nibble(uint8_t v)
{
    int x = v & 0x0F;
    return (int8_t)(x >= 8 ? x - 16 : x);
}

/* codes [N][K] -> N x packed-K [N][K/2]: byte j of row n holds codes 2j, 2j+1 */
int oracle_pack_nk(const int8_t* Q, int64_t N, int64_t K, uint8_t* P)
{
    if (N < 0 || K <= 0 || K % 2) return -1;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < K / 2; ++j)
            P[n * (K / 2) + j] = (uint8_t)(nibble(Q[n * K + 2 * j]) | (nibble(Q[n * K + 2 * j + 1]) << 4));
    return 0;
}

int oracle_unpack_nk(const uint8_t* P, int64_t N, int64_t K, int8_t* Q)
{
    if (N < 0 || K <= 0 || K % 2) return -1;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < K / 2; ++j) {
            uint8_t b = P[n * (K / 2) + j];
            Q[n * K + 2 * j] = from_nibble(b & 0x0F);
            Q[n * K + 2 * j + 1] = from_nibble(b >> 4);
        }
    return 0;
}

/* N x packed-K [N][K/2] -> K x packed-N [K][N/2]: byte j of row k holds the
 * codes of output channels 2j and 2j+1 at input channel k. */
int oracle_nk_to_kn(const uint8_t* P_nk, int64_t N, int64_t K, uint8_t* P_kn)
{
    if (N <= 0 || K <= 0 || N % 2 || K % 2) return -1;
    int8_t* Q = (int8_t*)malloc((size_t)N * (size_t)K);
    if (!Q) return -2;
    oracle_unpack_nk(P_nk, N, K, Q);
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N / 2; ++j)
            P_kn[k * (N / 2) + j] = (uint8_t)(nibble(Q[(2 * j) * K + k]) | (nibble(Q[(2 * j + 1) * K + k]) << 4));
    free(Q);
    return 0;
}

int oracle_kn_to_nk(const uint8_t* P_kn, int64_t N, int64_t K, uint8_t* P_nk)
{
    if (N <= 0 || K <= 0 || N % 2 || K % 2) return -1;
    int8_t* Q = (int8_t*)malloc((size_t)N * (size_t)K);
    if (!Q) return -2;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N / 2; ++j) {
            uint8_t b = P_kn[k * (N / 2) + j];
            Q[(2 * j) * K + k] = from_nibble(b & 0x0F);
            Q[(2 * j + 1) * K + k] = from_nibble(b >> 4);
        }
    oracle_pack_nk(Q, N, K, P_nk);
    free(Q);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* 5. Integer dot products acc[m][n] = sum_k qx[m][k] * qw[n][k]              */
/* ------------------------------------------------------------------------ */

struct gemm_ctx {
    const int8_t* QX;
    const int8_t* QW;
    int64_t N, K;
    int32_t* ACC;
    int overflow; /* set if any sum leaves the int32 range */
};

static void gemm_one_row(void* p, int64_t m)
{
    struct gemm_ctx* c = (struct gemm_ctx*)p;
    const int8_t* x = c->QX + m * c->K;
    for (int64_t n = 0; n < c->N; ++n) {
        const int8_t* w = c->QW + n * c->K;
        int64_t acc = 0;
        for (int64_t k = 0; k < c->K; ++k) acc += (int64_t)x[k] * (int64_t)w[k];
        if (acc > INT32_MAX || acc < INT32_MIN) c->overflow = 1;
        c->ACC[m * c->N + n] = (int32_t)acc;
    }
}

/* Returns 0, -1 on bad sizes, 1 if some sum does not fit int32. */
int oracle_gemm_i32(const int8_t* QX, const int8_t* QW, int64_t M, int64_t N, int64_t K, int32_t* ACC,
                    int nthreads)
{
    if (M < 0 || N < 0 || K <= 0) return -1;
    struct gemm_ctx c = {QX, QW, N, K, ACC, 0};
    parallel_rows(gemm_one_row, &c, M, nthreads);
    return c.overflow ? 1 : 0;
}

/* ------------------------------------------------------------------------ */
/* 6. Epilogue: y = bf16(fmaf(float(acc) * sx[m], sw[n], bias[n]))           */
/* ------------------------------------------------------------------------ */

/* The binary32 value that the epilogue rounds to bf16: the integer sum times
 * the row scale, rounded once, then one fused multiply-add with the column
 * scale and the bias (a single rounding). */
static float epilogue_value(int32_t acc, float sx, float sw, float b)
{
    float t = (float)acc * sx;
    return fmaf(t, sw, b);
}

/* bias: bf16 bits [N] or NULL for zeros.  Y: bf16 bits [M][N]; YF (may be
 * NULL): the binary32 values before the bf16 rounding. */
void oracle_epilogue_f32(const int32_t* ACC, const float* SX, const float* SW, const uint16_t* BIAS, int64_t M,
                         int64_t N, uint16_t* Y, float* YF)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            float b = BIAS ? oracle_bf16_to_f32(BIAS[n]) : 0.0f;
            float y = epilogue_value(ACC[m * N + n], SX[m], SW[n], b);
            if (YF) YF[m * N + n] = y;
            if (Y) Y[m * N + n] = oracle_f32_to_bf16(y);
        }
}

void oracle_epilogue(const int32_t* ACC, const float* SX, const float* SW, const uint16_t* BIAS, int64_t M,
                     int64_t N, uint16_t* Y)
{
    oracle_epilogue_f32(ACC, SX, SW, BIAS, M, N, Y, NULL);
}

/* ------------------------------------------------------------------------ */
/* 7. The whole linear, given prepared weight codes and scales               */
/* ------------------------------------------------------------------------ */

/* X: bf16 [M][K]; QW: int8 codes [N][K]; SW: [N]; BIAS: bf16 [N] or NULL.
 * Optional outputs QX_out [M][K_rot], SX_out [M], ACC_out [M][N] may be NULL.
 * QW is [N][K_rot] (weight rows prepared with the same g).  Returns 0 on
 * success. */
int oracle_linear(const uint16_t* X, int64_t M, int64_t K, const int8_t* QW, const float* SW,
                  const uint16_t* BIAS, int64_t N, int g, uint16_t* Y, int8_t* QX_out, float* SX_out,
                  int32_t* ACC_out, int nthreads)
{
    if (M < 0 || N < 0 || K <= 0) return -1;
    const int64_t Kr = oracle_rotated_width(K, g);
    size_t mk = (size_t)(M > 0 ? M : 1) * (size_t)Kr;
    size_t mn = (size_t)(M > 0 ? M : 1) * (size_t)(N > 0 ? N : 1);
    int8_t* QX = QX_out ? QX_out : (int8_t*)malloc(mk);
    float* SX = SX_out ? SX_out : (float*)malloc((size_t)(M > 0 ? M : 1) * sizeof(float));
    int32_t* ACC = ACC_out ? ACC_out : (int32_t*)malloc(mn * sizeof(int32_t));
    int rc = (!QX || !SX || !ACC) ? -2 : 0;
    if (rc == 0) rc = oracle_prepare_rows(X, M, K, g, QX, SX, NULL, nthreads);
    if (rc == 0) rc = oracle_gemm_i32(QX, QW, M, N, Kr, ACC, nthreads);
    if (rc == 0) oracle_epilogue(ACC, SX, SW, BIAS, M, N, Y);
    if (!QX_out) free(QX);
    if (!SX_out) free(SX);
    if (!ACC_out) free(ACC);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* 8. W4A16: rotated activations rounded to bf16, INT4 weight codes           */
/* ------------------------------------------------------------------------ */

struct w4a16_ctx {
    const uint16_t* XR; /* bf16 rotated activations [M][K] */
    const int8_t* QW;
    const float* SW;
    const uint16_t* BIAS;
    int64_t N, K;
    uint16_t* Y;
    float* YF; /* binary32 values before the bf16 rounding, or NULL */
};

static void w4a16_one_row(void* p, int64_t m)
{
    struct w4a16_ctx* c = (struct w4a16_ctx*)p;
    const uint16_t* x = c->XR + m * c->K;
    for (int64_t n = 0; n < c->N; ++n) {
        const int8_t* q = c->QW + n * c->K;
        double acc = 0.0; /* each product is exact; |sum| is far below 2^53 ulps of the terms */
        for (int64_t k = 0; k < c->K; ++k) acc += (double)oracle_bf16_to_f32(x[k]) * (double)q[k];
        float b = c->BIAS ? oracle_bf16_to_f32(c->BIAS[n]) : 0.0f;
        float y = fmaf((float)acc, c->SW[n], b); /* sum rounded once to binary32, then one fused multiply-add */
        if (c->YF) c->YF[m * c->N + n] = y;
        c->Y[m * c->N + n] = oracle_f32_to_bf16(y);
    }
}

/* X: bf16 [M][K]; QW: int8 codes [N][K_rot]; SW: [N]; BIAS: bf16 [N] or NULL;
 * Y: bf16 [M][N]; XR_out (optional): the bf16 rotated activations [M][K_rot];
 * YF_out (optional): the binary32 outputs before the bf16 rounding [M][N].
 * g as for oracle_rotate_rows.  Returns 0 on success. */
int oracle_linear_w4a16(const uint16_t* X, int64_t M, int64_t K, const int8_t* QW, const float* SW,
                        const uint16_t* BIAS, int64_t N, int g, uint16_t* Y, uint16_t* XR_out, float* YF_out,
                        int nthreads)
{
    if (M < 0 || N < 0 || K <= 0) return -1;
    const int64_t Kr = oracle_rotated_width(K, g);
    size_t mk = (size_t)(M > 0 ? M : 1) * (size_t)Kr;
    float* R = (float*)malloc(mk * sizeof(float));
    uint16_t* XR = XR_out ? XR_out : (uint16_t*)malloc(mk * sizeof(uint16_t));
    int rc = (!R || !XR) ? -2 : 0;
    if (rc == 0) rc = oracle_rotate_rows(X, M, K, g, R, nthreads);
    if (rc == 0) {
        for (size_t i = 0; i < (size_t)M * (size_t)Kr; ++i) XR[i] = oracle_f32_to_bf16(R[i]);
        struct w4a16_ctx c = {XR, QW, SW, BIAS, N, Kr, Y, YF_out};
        parallel_rows(w4a16_one_row, &c, M, nthreads);
    }
    free(R);
    if (!XR_out) free(XR);
    return rc;
}
