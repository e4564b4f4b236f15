// kernels.hip -- gfx950 (CDNA4) kernels of the ConvRot W4A4 linear.
//
//   prep_kernel   rotation (grouped Sylvester Hadamard, fast Walsh-Hadamard
//                 butterflies in fp32), row absmax, symmetric INT4
//                 quantization; writes codes in one of four layouts.
//   gemm_kernel   INT8 x INT4 GEMM on the INT8 matrix cores
//                 (v_mfma_i32_32x32x32_i8) with int32 accumulation and the
//                 scale + bias epilogue to bf16 (or raw int32 for parity).
//   repack_nk_kernel / act_relayout_kernel: lossless layout moves.
//
// Method: convrot-mlx README, "What is included" (normalized Hadamard
// rotation over groups of 64 or 256, symmetric rowwise absmax INT4 in
// [-7, 7], reversible packed layouts) and comfy-quants issue "convrot is ...
// QuaRot Stage 1c", section 1 (R = I_G (x) H, X.R = [X_1 H, ..., X_G H]).
#include <hip/hip_runtime.h>

#include "kernels.h"
#include "layout.h"

namespace convrot {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

// ---------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// binary32 -> bf16 bits, round to nearest even (finite values)
__device__ inline uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Value of lane (lane ^ m) for m = 1, 2 within a quad (DPP quad_perm), for a
// 64-bit value moved as two 32-bit halves.
template <int M>
__device__ inline double quad_xor(double v)
{
    constexpr int ctrl = (M == 1) ? 0xB1 /* [1,0,3,2] */ : 0x4E /* [2,3,0,1] */;
    const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), ctrl, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), ctrl, 0xF, 0xF, false);
    return __hiloint2double(hi, lo);
}

// Code = clamp(rint(fl32(r / s)), -7, 7).  Fast path: y = r * rcp(s) is within
// 2 ulp of r / s (|y| < 8, so 2 ulp <= 2^-20); whenever y is farther than
// 2^-18 from a half-integer, rint(y) equals rint(fl32(r / s)) because no
// rounding boundary lies between them.  Near a half-integer (or when s is not
// a normal number) the correctly rounded binary32 division decides.
__device__ inline int8_t quantize_one(float r, float s, float inv, bool exact_only)
{
    float q;
    const float y = r * inv;
    const float ry = rintf(y);
    if (exact_only || fabsf(fabsf(y - ry) - 0.5f) < 0x1p-18f)
        q = rintf(r / s);  // IEEE binary32 division, round half to even
    else
        q = ry;
    q = fminf(fmaxf(q, -7.0f), 7.0f);
    return (int8_t)q;
}

__device__ inline uint32_t nib(int8_t q) { return (uint32_t)(uint8_t)q & 0xFu; }

__device__ inline uint32_t pack4_i8(const int8_t* q)
{
    return (uint32_t)(uint8_t)q[0] | ((uint32_t)(uint8_t)q[1] << 8) | ((uint32_t)(uint8_t)q[2] << 16) |
           ((uint32_t)(uint8_t)q[3] << 24);
}

// ---------------------------------------------------------------------------
// prep_kernel
//
// Work split: a row is cut into 64-element "slices"; each lane owns one
// slice.  For g = 256 a group is 4 slices on 4 consecutive lanes (a quad):
// lane q of the quad holds group elements 8q + 32j + e (j, e = 0..7), so the
// butterflies over index bits 0-2 (e) and 5-7 (j) run in registers and the
// two over bits 3-4 (q) are quad DPP exchanges.  For g = 64 a group is one
// contiguous slice and all six butterfly stages run in registers.
// A "team" of lanes covers one row: team <= 64 lanes share a wave with other
// rows; team > 64 is a whole workgroup and reduces the row absmax via LDS.
//
// Precision: the butterflies run in binary64 (on gfx950 a double add issues
// at the rate of an unpacked float add) and each rotated value is rounded
// once to binary32.  A sum of g bf16 values whose magnitudes span fewer than
// ~37 binary orders is exact in binary64, so the binary32 value is the
// correctly rounded exact rotation and the codes do not depend on the
// butterfly order.
// ---------------------------------------------------------------------------

template <int G>
__device__ inline int64_t slice_k(int s, int j)
{
    if constexpr (G == 256)
        return (int64_t)(s >> 2) * 256 + 32 * j + 8 * (s & 3);
    else
        return (int64_t)s * 64 + 8 * j;
}

template <int G, int MODE>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs a)
{
    const int tid = threadIdx.x;
    int64_t row;
    int slice;
    if (a.team <= 64) {
        const int rows_per_block = blockDim.x / a.team;
        row = (int64_t)blockIdx.x * rows_per_block + tid / a.team;
        slice = tid % a.team;
    } else {
        row = blockIdx.x;
        slice = tid;
    }
    const bool row_in = row < a.rows_pad;           // lane has a row to write
    const bool row_valid = row < a.rows;            // row holds data
    const int spr = (int)(a.K / 64);                // slices holding data
    const bool has_data = row_valid && slice < spr;

    double v[8][8];
    {
        uint4 w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            w[j] = make_uint4(0, 0, 0, 0);
            if (has_data) w[j] = *(const uint4*)(a.X + row * a.K + slice_k<G>(slice, j));
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            v[j][0] = bf16_lo(w[j].x); v[j][1] = bf16_hi(w[j].x);
            v[j][2] = bf16_lo(w[j].y); v[j][3] = bf16_hi(w[j].y);
            v[j][4] = bf16_lo(w[j].z); v[j][5] = bf16_hi(w[j].z);
            v[j][6] = bf16_lo(w[j].w); v[j][7] = bf16_hi(w[j].w);
        }
    }

    // butterflies over e (index bits 0..2)
#pragma unroll
    for (int b = 1; b < 8; b <<= 1)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (!(e & b)) {
                    double x = v[j][e], y = v[j][e | b];
                    v[j][e] = x + y;
                    v[j][e | b] = x - y;
                }
    // butterflies over j (index bits 5..7 for g = 256, 3..5 for g = 64)
#pragma unroll
    for (int b = 1; b < 8; b <<= 1)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (!(j & b))
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    double x = v[j][e], y = v[j | b][e];
                    v[j][e] = x + y;
                    v[j | b][e] = x - y;
                }
    if constexpr (G == 256) {
        // butterflies over q (index bits 3..4): lane pairs (l, l^1), (l, l^2)
        const bool up1 = (tid & 1) != 0, up2 = (tid & 2) != 0;
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                double p = quad_xor<1>(v[j][e]);
                v[j][e] = up1 ? (p - v[j][e]) : (v[j][e] + p);
            }
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                double p = quad_xor<2>(v[j][e]);
                v[j][e] = up2 ? (p - v[j][e]) : (v[j][e] + p);
            }
    }
    constexpr double kNorm = (G == 256) ? 0.0625 : 0.125;  // 1/sqrt(g), exact
    float r[8][8];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            r[j][e] = (float)(v[j][e] * kNorm);  // the one rounding to binary32
            amax = fmaxf(amax, fabsf(r[j][e]));
        }

    // row absmax over the team
    if (a.team <= 64) {
        for (int o = 1; o < a.team; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    } else {
        __shared__ float red[16];
        for (int o = 1; o < 64; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
        if ((tid & 63) == 0) red[tid >> 6] = amax;
        __syncthreads();
        amax = red[0];
        for (int w = 1; w < (int)(blockDim.x >> 6); ++w) amax = fmaxf(amax, red[w]);
    }
    const bool zero_row = !(amax > 0.0f);
    const float s = zero_row ? 0.0f : amax / 7.0f;  // IEEE binary32 division
    const bool exact_only = !(s >= 0x1p-126f);      // s not a normal number
    const float inv = exact_only ? 0.0f : __builtin_amdgcn_rcpf(s);

    if (!row_in) return;
    if (row_valid && slice == 0) a.scales[row] = s;

    const bool write_slice = (MODE == OUT_ACT_IMAGE || MODE == OUT_WGT_IMAGE) ? (slice < a.slices_pad) : has_data;
    if (!write_slice) return;

#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int64_t k = slice_k<G>(slice, j);
        int8_t q[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = zero_row ? (int8_t)0 : quantize_one(r[j][e], s, inv, exact_only);
        if constexpr (MODE == OUT_ACT_IMAGE) {
            uint2 w;
            w.x = pack4_i8(q);
            w.y = pack4_i8(q + 4);
            *(uint2*)(a.out + act_chunk_offset(row, k & ~(int64_t)15, a.K_pad) + (k & 8)) = w;
        } else if constexpr (MODE == OUT_WGT_IMAGE) {
            uint32_t w = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) w |= (nib(q[b]) | (nib(q[b + 4]) << 4)) << (8 * b);
            *(uint32_t*)(a.out + wgt_word_offset(row, k, a.K_pad)) = w;
        } else if constexpr (MODE == OUT_NK) {
            uint32_t w = 0;
#pragma unroll
            for (int u = 0; u < 4; ++u) w |= (nib(q[2 * u]) | (nib(q[2 * u + 1]) << 4)) << (8 * u);
            *(uint32_t*)(a.out + row * (a.K / 2) + k / 2) = w;
        } else {  // OUT_ROWMAJOR
            uint2 w;
            w.x = pack4_i8(q);
            w.y = pack4_i8(q + 4);
            *(uint2*)(a.out + row * a.K + k) = w;
            if (a.rotated) {
                float4* rp = (float4*)(a.rotated + row * a.K + k);
                rp[0] = make_float4(r[j][0], r[j][1], r[j][2], r[j][3]);
                rp[1] = make_float4(r[j][4], r[j][5], r[j][6], r[j][7]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// gemm_kernel
//
// Block tile 256 (M) x 256 (N), K stepped 128 at a time through a double
// buffer in LDS: 8 activation units (4 KB each) + 8 weight units (2 KB each)
// = 48 KB per stage, copied global -> LDS with global_load_lds_dwordx4 (the
// images are stored in exactly the LDS order, so every copy is a straight
// 1 KB run per wave instruction).  Four waves in a 2 x 2 arrangement each own
// a 128 x 128 output tile = 4 x 4 MFMA 32x32x32 tiles.  Weight nibbles are
// widened to INT8 x 16 in registers right after the LDS read; the int32
// accumulators are divided by 16 (exact) in the epilogue.
// ---------------------------------------------------------------------------

constexpr int kBM = 256, kBN = 256;
constexpr int kStageA = 8 * kActUnitBytes;   // 32 KB
constexpr int kStageB = 8 * kWgtUnitBytes;   // 16 KB
constexpr int kStage = kStageA + kStageB;    // 48 KB

// Global -> register half of a stage copy: each wave moves 8 KB of
// activation units and 4 KB of weight units, 16 bytes per lane per load.
struct StageRegs {
    uint4 a[8];
    uint4 b[4];
};

__device__ inline void load_stage(const GemmArgs& a, StageRegs& st, int mt0, int nt0, int kb, int wave, int lane)
{
#pragma unroll
    for (int u2 = 0; u2 < 2; ++u2) {
        const int mt = mt0 + 2 * wave + u2;
        const uint8_t* src = a.act + ((size_t)mt * a.KB + kb) * kActUnitBytes + lane * 16;
        const bool ok = mt < a.MT;
#pragma unroll
        for (int p = 0; p < 4; ++p)
            st.a[u2 * 4 + p] = ok ? *(const uint4*)(src + p * 1024) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u2 = 0; u2 < 2; ++u2) {
        const int nt = nt0 + 2 * wave + u2;
        const uint8_t* src = a.wgt + ((size_t)nt * a.KB + kb) * kWgtUnitBytes + lane * 16;
        const bool ok = nt < a.NT;
#pragma unroll
        for (int p = 0; p < 2; ++p)
            st.b[u2 * 2 + p] = ok ? *(const uint4*)(src + p * 1024) : make_uint4(0, 0, 0, 0);
    }
}

// Register -> LDS half: the images are stored in LDS order, so lane l of a
// wave writes bytes [16 l, 16 l + 16) of each 1 KB piece.
__device__ inline void store_stage(uint8_t* stage, const StageRegs& st, int wave, int lane)
{
#pragma unroll
    for (int u2 = 0; u2 < 2; ++u2)
#pragma unroll
        for (int p = 0; p < 4; ++p)
            *(uint4*)(stage + (2 * wave + u2) * kActUnitBytes + p * 1024 + lane * 16) = st.a[u2 * 4 + p];
#pragma unroll
    for (int u2 = 0; u2 < 2; ++u2)
#pragma unroll
        for (int p = 0; p < 2; ++p)
            *(uint4*)(stage + kStageA + (2 * wave + u2) * kWgtUnitBytes + p * 1024 + lane * 16) = st.b[u2 * 2 + p];
}

__device__ inline v4i widen_lo_hi(uint32_t w0, uint32_t w1)
{
    v4i r;
    r[0] = (int)((w0 << 4) & 0xF0F0F0F0u);
    r[1] = (int)(w0 & 0xF0F0F0F0u);
    r[2] = (int)((w1 << 4) & 0xF0F0F0F0u);
    r[3] = (int)(w1 & 0xF0F0F0F0u);
    return r;
}

// One 128-K stage of MFMAs out of LDS.  Fragments for the next k-step are
// read before the current k-step's MFMAs are issued.
__device__ inline void compute_stage(const uint8_t* stage, int wm, int wn, int r32, int h, v16i (&acc)[4][4])
{
    const uint8_t* sa = stage + (wm * 4) * kActUnitBytes + r32 * 128;
    const uint8_t* sb = stage + kStageA + (wn * 4) * kWgtUnitBytes + r32 * 64;
    const int swz_a = r32 & 7, swz_b = (r32 >> 1) & 3;
    uint4 bq[2][4];
    v4i af[2][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bq[0][j] = *(const uint4*)(sb + j * kWgtUnitBytes + ((h ^ swz_b) * 16));
#pragma unroll
    for (int i = 0; i < 4; ++i) af[0][i] = *(const v4i*)(sa + i * kActUnitBytes + ((h ^ swz_a) * 16));
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const int cur = ks & 1, nxt = cur ^ 1;
        if (ks + 1 < 4) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[nxt][i] = *(const v4i*)(sa + i * kActUnitBytes + (((2 * (ks + 1) + h) ^ swz_a) * 16));
        }
        if (ks == 1) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bq[1][j] = *(const uint4*)(sb + j * kWgtUnitBytes + (((2 + h) ^ swz_b) * 16));
        }
        const int pr = ks >> 1;
        v4i bf[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            bf[j] = (ks & 1) == 0 ? widen_lo_hi(bq[pr][j].x, bq[pr][j].y) : widen_lo_hi(bq[pr][j].z, bq[pr][j].w);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[cur][i], bf[j], acc[i][j], 0, 0, 0);
    }
}

template <int OUT>
__global__ __launch_bounds__(256, 1) void gemm_kernel(GemmArgs a)
{
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kStage];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // XCD-aware tile order: workgroup i runs on XCD i % 8; give each XCD a
    // contiguous range of tiles (row tiles fastest) so tiles sharing weight
    // columns share that XCD's L2.
    const int total = a.tiles_m * a.tiles_n;
    const int wg = blockIdx.x;
    const int qx = total / 8, rx = total % 8;
    const int xcd = wg % 8, idx = wg / 8;
    const int vid = xcd * qx + (xcd < rx ? xcd : rx) + idx;
    const int tm = vid % a.tiles_m, tn = vid / a.tiles_m;
    const int mt0 = tm * (kBM / 32), nt0 = tn * (kBN / 32);

    v16i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    const int r32 = lane & 31, h = lane >> 5;

    StageRegs st;
    load_stage(a, st, mt0, nt0, 0, wave, lane);
    store_stage(smem, st, wave, lane);
    __syncthreads();

    for (int kb = 0; kb < a.KB; ++kb) {
        const bool more = kb + 1 < a.KB;
        if (more) load_stage(a, st, mt0, nt0, kb + 1, wave, lane);  // in flight during the MFMAs
        compute_stage(smem + (kb & 1) * kStage, wm, wn, r32, h, acc);
        if (more) store_stage(smem + ((kb + 1) & 1) * kStage, st, wave, lane);
        __syncthreads();
    }

    // epilogue: D[i][j] of a 32x32 MFMA tile sits in lane (j + 32 * ((i / 4) % 2)),
    // register (i / 8) * 4 + i % 4.
    const int64_t m_base = (int64_t)tm * kBM + wm * 128;
    const int64_t n_base = (int64_t)tn * kBN + wn * 128;
    float swn[4], bn[4];
    bool n_ok[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t n = n_base + 32 * j + r32;
        n_ok[j] = n < a.N;
        swn[j] = 0.0f;
        bn[j] = 0.0f;
        if (OUT == GEMM_OUT_BF16 && n_ok[j]) {
            swn[j] = a.sw[n];
            bn[j] = a.bias ? __uint_as_float((uint32_t)a.bias[n] << 16) : 0.0f;
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t m = m_base + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
            if (m >= a.M) continue;
            const float sxm = (OUT == GEMM_OUT_BF16) ? a.sx[m] : 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (!n_ok[j]) continue;
                const int64_t n = n_base + 32 * j + r32;
                const int32_t v = acc[i][j][r] >> 4;  // weights entered as 16 * code
                if constexpr (OUT == GEMM_OUT_I32) {
                    ((int32_t*)a.out)[m * a.N + n] = v;
                } else {
                    const float t = (float)v * sxm;
                    const float y = __builtin_fmaf(t, swn[j], bn[j]);
                    ((uint16_t*)a.out)[m * a.N + n] = f32_to_bf16_rne(y);
                }
            }
        }
}

// ---------------------------------------------------------------------------
// layout kernels
// ---------------------------------------------------------------------------

// int8 codes [M][K] -> activation image (zero padding); one thread per 16 codes.
__global__ void act_relayout_kernel(const int8_t* codes, int64_t M, int64_t K, int64_t M_pad, int64_t K_pad,
                                    uint8_t* image)
{
    const int64_t chunks_per_row = K_pad / 16;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= M_pad * chunks_per_row) return;
    const int64_t m = t / chunks_per_row, k = (t % chunks_per_row) * 16;
    uint4 w = make_uint4(0, 0, 0, 0);
    if (m < M && k < K) w = *(const uint4*)(codes + m * K + k);
    *(uint4*)(image + act_chunk_offset(m, k, K_pad)) = w;
}

// N x packed-K [N][K/2] -> weight image (zero padding); one thread per 8 codes.
__global__ void repack_nk_kernel(const uint8_t* nk, int64_t N, int64_t K, int64_t N_pad, int64_t K_pad,
                                 uint8_t* image)
{
    const int64_t words_per_col = K_pad / 8;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= N_pad * words_per_col) return;
    const int64_t n = t / words_per_col, k = (t % words_per_col) * 8;
    uint32_t out = 0;
    if (n < N && k < K) {
        const uint32_t in = *(const uint32_t*)(nk + n * (K / 2) + k / 2);  // codes k..k+7, two per byte
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint32_t c_lo = (in >> (4 * b)) & 0xFu;        // code k + b
            const uint32_t c_hi = (in >> (4 * (b + 4))) & 0xFu;  // code k + 4 + b
            out |= (c_lo | (c_hi << 4)) << (8 * b);
        }
    }
    *(uint32_t*)(image + wgt_word_offset(n, k, K_pad)) = out;
}

// ---------------------------------------------------------------------------
// host-side launchers
// ---------------------------------------------------------------------------

template <int G, int MODE>
static void launch_prep_g(const PrepArgs& a, dim3 grid, dim3 block, hipStream_t s)
{
    hipLaunchKernelGGL((prep_kernel<G, MODE>), grid, block, 0, s, a);
}

template <int MODE>
static void launch_prep_mode(int g, const PrepArgs& a, dim3 grid, dim3 block, hipStream_t s)
{
    if (g == 256)
        launch_prep_g<256, MODE>(a, grid, block, s);
    else
        launch_prep_g<64, MODE>(a, grid, block, s);
}

void launch_prep(int g, int mode, PrepArgs a, hipStream_t s)
{
    const int slices_pad = (int)(a.K_pad / 64);
    int team = 1;
    if (slices_pad <= 64) {
        while (team < slices_pad) team <<= 1;
    } else {
        team = (slices_pad + 63) / 64 * 64;
    }
    a.team = team;
    a.slices_pad = slices_pad;
    dim3 block, grid;
    if (team <= 64) {
        block = dim3(256);
        const int64_t rows_per_block = 256 / team;
        grid = dim3((unsigned)((a.rows_pad + rows_per_block - 1) / rows_per_block));
    } else {
        block = dim3(team);
        grid = dim3((unsigned)a.rows_pad);
    }
    switch (mode) {
        case OUT_ACT_IMAGE: launch_prep_mode<OUT_ACT_IMAGE>(g, a, grid, block, s); break;
        case OUT_WGT_IMAGE: launch_prep_mode<OUT_WGT_IMAGE>(g, a, grid, block, s); break;
        case OUT_NK: launch_prep_mode<OUT_NK>(g, a, grid, block, s); break;
        default: launch_prep_mode<OUT_ROWMAJOR>(g, a, grid, block, s); break;
    }
}

void launch_gemm(int out_mode, GemmArgs a, hipStream_t s)
{
    a.tiles_m = (a.MT + kBM / 32 - 1) / (kBM / 32);
    a.tiles_n = (a.NT + kBN / 32 - 1) / (kBN / 32);
    dim3 grid((unsigned)(a.tiles_m * a.tiles_n)), block(256);
    if (out_mode == GEMM_OUT_I32)
        hipLaunchKernelGGL((gemm_kernel<GEMM_OUT_I32>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((gemm_kernel<GEMM_OUT_BF16>), grid, block, 0, s, a);
}

void launch_act_relayout(const int8_t* codes, int64_t M, int64_t K, uint8_t* image, hipStream_t s)
{
    const int64_t M_pad = round_up(M, kTileRows), K_pad = round_up(K, kTileK);
    const int64_t n = M_pad * (K_pad / 16);
    hipLaunchKernelGGL(act_relayout_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, codes, M, K, M_pad,
                       K_pad, image);
}

void launch_repack_nk(const uint8_t* nk, int64_t N, int64_t K, uint8_t* image, hipStream_t s)
{
    const int64_t N_pad = round_up(N, kTileRows), K_pad = round_up(K, kTileK);
    const int64_t n = N_pad * (K_pad / 8);
    hipLaunchKernelGGL(repack_nk_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, nk, N, K, N_pad, K_pad,
                       image);
}

}  // namespace convrot
