// kernels.hip -- gfx950 (CDNA4) kernels of the ConvRot W4A4 linear.
//
//   prep_kernel   rotation (grouped Sylvester or regular Hadamard as fast
//                 Walsh-Hadamard butterflies in binary64, rounded once to
//                 binary32), row absmax, symmetric INT4 quantization; writes
//                 the codes as the operand images (INT4, and FP6 e2m3 for
//                 the FP6 matrix cores), in plain layouts for parity checks,
//                 or the rotated rows as bf16 (W4A16).
//   gemm6_kernel  the block-tile product on the FP6 matrix cores
//                 (v_mfma_scale_f32_32x32x64_f8f6f4: the codes are exact
//                 e2m3 values, the binary32 sums exact integers) with the
//                 scale + bias epilogue to bf16 (or int32 for parity).
//   gemm_kernel   the same on the INT8 matrix cores (v_mfma_i32_32x32x32_i8,
//                 codes widened to INT8 x 16 in registers), two tile shapes,
//                 one of them split along K.
//   skinny_kernel the weight-streaming product of M <= 128.
//   small_m_kernel, w4a16_kernel, small_w4a16_kernel:
//                 one-launch W4A4 for M <= 4 (the rows rotated in every
//                 workgroup) and the weight-only variant (M <= 32).
//   relayout kernels: lossless layout moves into the operand images.
//
// Method: convrot-mlx README, "What is included" (normalized Hadamard
// rotation over groups of 64 or 256, symmetric rowwise absmax INT4 in
// [-7, 7], reversible packed layouts) and comfy-quants issue "convrot is ...
// QuaRot Stage 1c", section 1 (R = I_G (x) H, X.R = [X_1 H, ..., X_G H]).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>

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

// Two binary32 -> two bf16 (round to nearest even) packed low | high << 16:
// one v_cvt_pk_bf16_f32 on gfx950.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pack_bf16x2(float lo, float hi)
{
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Codes = clamp(rint(fl32(r / s)), -7, 7) for the P values of a lane, each
// returned as the bit pattern of the binary32 value 1.5 * 2^23 + code, whose
// low byte is the code in two's complement (adding 1.5 * 2^23 to |y| < 2^22
// rounds y to an integer, ties to even, held in the low mantissa bits).
// Fast path: y = r * rcp(s) is within 2 ulp of r / s (|y| < 8, so the error is
// below 2^-20); whenever y is farther than 2^-18 from a half-integer, rint(y)
// equals rint(fl32(r / s)) because no rounding boundary lies between them.
// The residual y - rint(y) is exact, so the test is exact.  Elements near a
// half-integer (and rows whose s is not a normal number) take the correctly
// rounded binary32 division, in a branch that is skipped unless some lane of
// the wave needs it.  With a normal s, |r| <= 7 s (1 + 2^-23) keeps every
// code in [-7, 7]; the clamp matters only on the division path, where a
// subnormal s can be far from absmax / 7.
template <int P>
__device__ inline void quantize_bits(const float (&r)[P], float s, bool zero_row, uint32_t (&f)[P])
{
    constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
    const bool exact_only = !(s >= 0x1p-126f);
    const float inv = exact_only ? 0.0f : __builtin_amdgcn_rcpf(s);
    float dmax = 0.0f;  // the largest distance to the rounded value (one compare for all P)
#pragma unroll
    for (int e = 0; e < P; ++e) {
        const float y = r[e] * inv;
        const float fy = y + kMagic;
        dmax = fmaxf(dmax, fabsf(y - (fy - kMagic)));
        f[e] = __float_as_uint(fy);
    }
    const bool need = exact_only || dmax > 0.5f - 0x1p-18f;
    if (need && !zero_row) {
#pragma unroll
        for (int e = 0; e < P; ++e) {
            const float y = r[e] * inv;
            const float fy = y + kMagic;
            if (exact_only || fabsf(y - (fy - kMagic)) > 0.5f - 0x1p-18f)
                f[e] = __float_as_uint(fminf(fmaxf(r[e] / s, -7.0f), 7.0f) + kMagic);  // IEEE division
        }
    }
    if (zero_row) {
#pragma unroll
        for (int e = 0; e < P; ++e) f[e] = __float_as_uint(kMagic);
    }
}

// Low bytes of four words, as bytes 0..3 of one word (v_perm_b32 selects bytes
// of the pair {hi, lo}: selectors 0-3 pick bytes of lo, 4-7 of hi, 12 gives 0).
__device__ inline uint32_t low_bytes4(uint32_t f0, uint32_t f1, uint32_t f2, uint32_t f3)
{
    return __builtin_amdgcn_perm(f1, f0, 0x0C0C0400u) | __builtin_amdgcn_perm(f3, f2, 0x04000C0Cu);
}

// One image word from the quantized bit patterns of codes k .. k+7: byte b
// holds code k+b in its low nibble and code k+4+b in its high nibble.
__device__ inline uint32_t image_word(const uint32_t* f)
{
    const uint32_t lo = low_bytes4(f[0], f[1], f[2], f[3]);
    const uint32_t hi = low_bytes4(f[4], f[5], f[6], f[7]);
    return (lo & 0x0F0F0F0Fu) | ((hi << 4) & 0xF0F0F0F0u);
}

// The FP6 (e2m3) fields of P = 8 or 16 codes, six bits each in code order, in
// the low 6 P bits of the result.  The hardware conversion takes two sets of
// 16 binary32 values and interleaves them (field 2i from the first set, 2i + 1
// from the second), so the even codes go in the first set and the odd codes in
// the second; the slots past P / 2 only feed fields that are not kept.  The
// inputs are the integer codes themselves (1.5 * 2^23 + code minus 1.5 * 2^23,
// exact), so the conversion with unit scale is exact.
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x6_t __attribute__((ext_vector_type(6)));
template <int P>
__device__ inline u32x6_t fp6_fields(const uint32_t (&f)[P])
{
    constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
    f32x16_t ev = __builtin_nondeterministic_value(ev), od = __builtin_nondeterministic_value(od);
#pragma unroll
    for (int i = 0; i < P / 2; ++i) {
        ev[i] = __uint_as_float(f[2 * i]) - kMagic;
        od[i] = __uint_as_float(f[2 * i + 1]) - kMagic;
    }
    return __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(ev, od, 1.0f);
}

// Max over a wave-row of DPP lanes.
template <int CTRL>
__device__ inline uint32_t max_dpp(uint32_t v)
{
    return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false));
}

// Max over the lanes of a team (8, 16 or 32 aligned lanes, or the whole wave
// when team >= 64) of the bit patterns of non-negative floats, which order as
// unsigned integers.
__device__ inline uint32_t team_max(uint32_t v, int team)
{
    v = max_dpp<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
    v = max_dpp<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
    v = max_dpp<0x141>(v);  // row_half_mirror: lanes i and 7 - i of each 8
    if (team >= 16) v = max_dpp<0x140>(v);  // row_mirror: lanes i and 15 - i of each 16
    if (team == 32) v = max(v, (uint32_t)__shfl_xor((int)v, 16, 64));
    if (team >= 64) {
        const uint32_t a0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
        const uint32_t a1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
        const uint32_t a2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
        const uint32_t a3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
        v = max(max(a0, a1), max(a2, a3));
    }
    return v;
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
// The g-point Sylvester transform factors as H_g = H_P (x) H_P with P = 16
// (g = 256) or P = 8 (g = 64): within a group, index u = P * hi + lo, and the
// butterflies over the bits of lo and over the bits of hi commute.  So:
//   phase 1: lane t owns the P consecutive elements t*P .. t*P + P - 1 of its
//            row (lo varies) and runs log2 P butterfly stages in registers;
//   transpose through LDS (within the wave: a group is P consecutive lanes);
//   phase 2: lane owns the P elements lo + P * hi (hi varies) of one group and
//            runs the other log2 P stages in registers.
// The butterflies run in binary64 (a double add issues at the rate of an
// unpacked float add on gfx950) and each value is rounded once to binary32; a
// sum of g bf16 values whose magnitudes span fewer than ~37 binary orders is
// exact in binary64, so the binary32 result is the correctly rounded exact
// rotation whatever the butterfly order.  The rotated values go back through
// LDS to phase-1 order, where the row absmax, the quantization and the packing
// of 8 consecutive codes per 32-bit word happen.
// A "team" of lanes covers one row (team = K_pad / P): teams of <= 64 lanes
// share waves; larger teams are a whole workgroup and reduce the absmax via
// LDS.
// ---------------------------------------------------------------------------

template <int G>
struct PrepShape {
    static constexpr int P = (G == 256) ? 16 : 8;             // elements per lane per phase
    static constexpr int kRunD = P + 2;                        // doubles per padded P-run in LDS
    static constexpr int kRunF = P + 4;                        // floats per padded P-run in LDS
    static constexpr int kWaveLdsBytes =                       // LDS per wave
        (32 * kRunD * 8 > 64 * kRunF * 4) ? 32 * kRunD * 8 : 64 * kRunF * 4;
};

// Loads of the P bf16 values of a lane's phase-1 run, in 16-byte chunks of 8
// values.  A row of X holds ld values (ld % 8 == 0); chunks past it are the
// zero padding of the last group.  The loads are always issued (from row 0,
// element 0 for a chunk without data -- a valid address) and such chunks are
// replaced by zeros (zero_unless), so the number of loads in flight is the
// same on every path and the wait for a prefetched row does not have to drain
// the newer loads.
template <int P>
__device__ inline void load_run(const uint16_t* X, int64_t row, int64_t ld, int64_t k0, bool has_row,
                                uint4 (&w)[P / 8])
{
#pragma unroll
    for (int c = 0; c < P / 8; ++c) {
        const bool ok = has_row && k0 + 8 * c < ld;
        w[c] = *(const uint4*)(X + (ok ? row * ld + k0 + 8 * c : 0));
    }
}

template <int P>
__device__ inline void zero_unless(bool has_row, int64_t ld, int64_t k0, uint4 (&w)[P / 8])
{
#pragma unroll
    for (int c = 0; c < P / 8; ++c)
        if (!(has_row && k0 + 8 * c < ld)) w[c] = make_uint4(0, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Regular Hadamard rotation.  The order-4 regular matrix B = J_4 - 2 I_4 is
// Pi D H_4 D, with H_4 the order-4 Sylvester matrix, D = diag(1, 1, 1, -1) and
// Pi the exchange of rows 0 and 3; so its k-th Kronecker power, the regular
// matrix of order g = 4^k, is (Pi D)^(x k) H_g D^(x k).  Rotating a group x by
// it is therefore: flip the sign of x_j when the base-4 digits of j hold an
// odd number of 3s (D^(x k)), apply the Sylvester butterflies, and take output
// o from Sylvester output pi(o), pi exchanging digits 0 and 3 in every base-4
// position, with the sign flipped when o has an odd number of 0 digits
// ((Pi D)^(x k)).  Sign flips and permutations are exact, so the rounded
// result is as exact as the Sylvester one.
// ---------------------------------------------------------------------------

// parity of the number of base-4 digits equal to 3 in x
__host__ __device__ constexpr uint32_t threes_parity(uint32_t x)
{
    return (uint32_t)__builtin_popcount(x & (x >> 1) & 0x55555555u) & 1u;
}

__device__ inline double negate_if(double v, uint32_t neg)
{
    return __hiloint2double(__double2hiint(v) ^ (int)(neg << 31), __double2loint(v));
}

__device__ inline float negate_if(float v, uint32_t neg) { return __uint_as_float(__float_as_uint(v) ^ (neg << 31)); }

// D^(x k) on the P inputs k0 .. k0 + P - 1 of a lane (k0 a multiple of P).
// With P = 16 the lane's two low digits are its own; with P = 8 digit 1 is
// split between bit 2 of the element and bit 3 of k0.
template <int G, int P>
__device__ inline void regular_input_signs(int64_t k0, double (&v)[P])
{
    const uint32_t hi = (uint32_t)(k0 % G);
    const uint32_t l0 = threes_parity(hi), l4 = threes_parity(hi | 4u);
#pragma unroll
    for (int e = 0; e < P; ++e) {
        const uint32_t neg = (P == 16) ? (l0 ^ threes_parity((uint32_t)e))
                                       : (((e & 4) ? l4 : l0) ^ threes_parity((uint32_t)(e & 3)));
        v[e] = negate_if(v[e], neg);
    }
}

// (Pi D)^(x k) on the way back to phase-1 order: lf holds this lane group's
// normalized Sylvester outputs z in natural order (z[i] at row i / P, column
// i % P of the group's rows starting at gbase).  Output o = 4 c + d of the
// lane takes z[4 pi(c) + pi(d)], pi(d) = 3, 1, 2, 0 for d = 0 .. 3, with the
// sign of (-1)^(zero digits of c) and one more flip for d == 0.
template <int G, int P, int RUN>
__device__ inline void regular_output_permutation(const float* lf, int gbase, int64_t k0, float (&r)[P])
{
    constexpr uint32_t kDigits = (G == 256) ? 3 : 2;              // base-4 digits of a block index c
    constexpr uint32_t kLow = 0x55555555u & ((1u << (2 * kDigits)) - 1);
    const uint32_t c0 = (uint32_t)(k0 % G) >> 2;                  // block index of the lane's first output
#pragma unroll
    for (int b = 0; b < P / 4; ++b) {
        const uint32_t c = c0 + (uint32_t)b;
        const uint32_t same = ~(c ^ (c >> 1)) & kLow;               // digits 0 or 3
        const uint32_t pc = c ^ (same | (same << 1));
        const uint32_t zpar = (uint32_t)__builtin_popcount(~(c | (c >> 1)) & kLow) & 1u;
        const uint32_t src = 4 * pc;
        const float4 q = *(const float4*)(lf + (gbase + (int)(src / P)) * RUN + (int)(src % P));
        r[4 * b + 0] = negate_if(q.w, zpar ^ 1u);
        r[4 * b + 1] = negate_if(q.y, zpar);
        r[4 * b + 2] = negate_if(q.z, zpar);
        r[4 * b + 3] = negate_if(q.x, zpar);
    }
}

// One row of the prep kernel: rotation, absmax, quantization and the write
// of the codes in the layout of MODE.  w holds the lane's P bf16 values.
// A team of more than 64 lanes is waves team_w0 .. team_w0 + team_nw - 1 of
// the workgroup.  OUT_LDS writes the image rows of a small row block into
// shared memory: row r of 128-K unit kb at ((kb * LDS_ROWS + r) * 64) with
// the image's in-row layout.
template <int G, int MODE, int LDS_ROWS = 0, bool REG = false>
__device__ __forceinline__ void prep_row(const PrepArgs& a, uint4 (&w)[PrepShape<G>::P / 8], int64_t row, int t,
                                         int64_t k0, int lane, int wave, double* ld, uint32_t (*red)[16], int parity,
                                         int team_w0, int team_nw)
{
    using S = PrepShape<G>;
    constexpr int P = S::P;
    const int gbase = (lane / P) * P;  // first lane of this lane's group
    const int lo = lane % P;           // phase-2: this lane's position in the low bits
    float* lf = (float*)ld;
    const bool row_valid = row < a.rows;  // row holds data
    const bool has_data = row_valid && k0 < a.K;
    // ---- phase 1: P consecutive elements, butterflies over the low bits ----
    zero_unless<P>(row_valid, a.ld, k0, w);
    double v[P];
#pragma unroll
    for (int c = 0; c < P / 8; ++c) {
        v[8 * c + 0] = bf16_lo(w[c].x); v[8 * c + 1] = bf16_hi(w[c].x);
        v[8 * c + 2] = bf16_lo(w[c].y); v[8 * c + 3] = bf16_hi(w[c].y);
        v[8 * c + 4] = bf16_lo(w[c].z); v[8 * c + 5] = bf16_hi(w[c].z);
        v[8 * c + 6] = bf16_lo(w[c].w); v[8 * c + 7] = bf16_hi(w[c].w);
    }
    if constexpr (REG) regular_input_signs<G, P>(k0, v);
#pragma unroll
    for (int b = 1; b < P; b <<= 1)
#pragma unroll
        for (int e = 0; e < P; ++e)
            if (!(e & b)) {
                const double x = v[e], y = v[e | b];
                v[e] = x + y;
                v[e | b] = x - y;
            }

    // ---- transpose through this wave's LDS region, half a group at a time ----
    // Pass hh: the lanes holding runs hh*P/2 .. hh*P/2 + P/2 - 1 of each
    // group write their P values to slot (group, run - hh*P/2); then every
    // lane reads element lo of those P/2 runs.  Half the region of a
    // whole-wave transpose; the padding keeps the 16-byte writes and the
    // 8-byte reads free of bank conflicts.
    double u[P];
    {
        const int slot_base = (lane / P) * (P / 2);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            if (lo / (P / 2) == hh) {
                double* dst = ld + (slot_base + lo % (P / 2)) * S::kRunD;
#pragma unroll
                for (int e = 0; e < P; e += 2) *(double2*)(dst + e) = make_double2(v[e], v[e + 1]);
            }
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
#pragma unroll
            for (int i = 0; i < P / 2; ++i) u[hh * (P / 2) + i] = ld[(slot_base + i) * S::kRunD + lo];
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_s_waitcnt(0xC07F);  // every lane's reads are done before the region is rewritten
            __builtin_amdgcn_wave_barrier();
        }
    }

    // ---- phase 2: butterflies over the high bits ----
#pragma unroll
    for (int b = 1; b < P; b <<= 1)
#pragma unroll
        for (int i = 0; i < P; ++i)
            if (!(i & b)) {
                const double x = u[i], y = u[i | b];
                u[i] = x + y;
                u[i | b] = x - y;
            }

    // ---- round once to binary32, back to phase-1 order through LDS ----
    constexpr double kNorm = (G == 256) ? 0.0625 : 0.125;  // 1/sqrt(g), exact
#pragma unroll
    for (int i = 0; i < P; ++i) lf[(gbase + i) * S::kRunF + lo] = (float)(u[i] * kNorm);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0xC07F);
    float r[P];
    if constexpr (!REG) {
#pragma unroll
        for (int e = 0; e < P; e += 4) {
            const float4 q = *(const float4*)(lf + lane * S::kRunF + e);
            r[e] = q.x; r[e + 1] = q.y; r[e + 2] = q.z; r[e + 3] = q.w;
        }
    } else {
        regular_output_permutation<G, P, S::kRunF>(lf, gbase, k0, r);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0xC07F);  // reads done before the next row rewrites the region
    __builtin_amdgcn_wave_barrier();

    // W4A16: the rotated row, rounded to bf16 (nearest even); no scale and
    // no codes.  K % 64 == 0, so every lane's P values are whole 16-byte
    // words: in the matrix-core order of w16_word_offset in device memory,
    // or row-major (rows K values apart) when LDS_ROWS > 0 (shared memory).
    if constexpr (MODE == OUT_ROTATED_BF16) {
        if (has_data) {
#pragma unroll
            for (int c = 0; c < P / 8; ++c) {
                const uint4 wd = make_uint4(pack_bf16x2(r[8 * c], r[8 * c + 1]), pack_bf16x2(r[8 * c + 2], r[8 * c + 3]),
                                            pack_bf16x2(r[8 * c + 4], r[8 * c + 5]),
                                            pack_bf16x2(r[8 * c + 6], r[8 * c + 7]));
                const size_t off = LDS_ROWS > 0 ? ((size_t)row * a.K + k0 + 8 * c) * 2
                                                : w16_word_offset(row, k0 + 8 * c, a.K);
                *(uint4*)(a.out + off) = wd;
            }
        }
        return;
    }

    // ---- row absmax over the team ----
    float lane_max = 0.0f;
#pragma unroll
    for (int e = 0; e < P; ++e) lane_max = fmaxf(lane_max, fabsf(r[e]));
    uint32_t amax_bits = team_max(__float_as_uint(lane_max), a.team);
    if (a.team > 64) {
        // red[parity] is rewritten two rows later, after every wave has
        // passed the next row's barrier (and so has read it)
        if (lane == 0) red[parity][wave] = amax_bits;
        __syncthreads();
        amax_bits = red[parity][team_w0];
        for (int wv = 1; wv < team_nw; ++wv) amax_bits = max(amax_bits, red[parity][team_w0 + wv]);
    }
    const float amax = __uint_as_float(amax_bits);
    const bool zero_row = !(amax > 0.0f);
    const float s = zero_row ? 0.0f : amax / 7.0f;  // IEEE binary32 division

    if (row_valid && t == 0) a.scales[row] = s;
    const bool write = (MODE == OUT_IMAGE || MODE == OUT_LDS) ? (k0 < a.K_pad && row < a.rows_pad) : has_data;
    if (write) {
        uint32_t f[P];
        quantize_bits<P>(r, s, zero_row, f);
        if constexpr (MODE == OUT_IMAGE) {
            // P/8 words for k0, k0 + 8 (adjacent dwords of one 8-byte group when P = 16)
            uint8_t* dst = a.out + image_word_offset(row, k0, a.K_pad);
            if (a.out) {
                if constexpr (P == 16)
                    *(uint2*)dst = make_uint2(image_word(f), image_word(f + 8));
                else
                    *(uint32_t*)dst = image_word(f);
            }
            if (a.out6) {
                // the same codes into the FP6 image: 6 P bits from logical
                // byte 24 (k0 % 128 / 32) + 6 P / 8 (k0 % 32 / P) of the row
                const u32x6_t fp = fp6_fields<P>(f);
                const int64_t kb = k0 / kTileK;
                const int kl = (int)(k0 % kTileK);
                const int b0 = 24 * (kl / 32) + (6 * P / 8) * ((kl % 32) / P);
                if constexpr (P == 16) {
                    // 12 bytes inside one 24-byte block: contiguous after the swizzle
                    *(uint3*)(a.out6 + image6_byte_offset(row, kb, b0, a.K_pad)) = make_uint3(fp[0], fp[1], fp[2]);
                } else {
                    const uint16_t hw[3] = {(uint16_t)fp[0], (uint16_t)(fp[0] >> 16), (uint16_t)fp[1]};
#pragma unroll
                    for (int d = 0; d < 3; ++d)
                        *(uint16_t*)(a.out6 + image6_byte_offset(row, kb, b0 + 2 * d, a.K_pad)) = hw[d];
                }
            }
        } else if constexpr (MODE == OUT_LDS) {
            const size_t unit_off = image_word_offset(row, k0, a.K_pad) % kUnitBytes;  // in-unit offset of row, k0
            uint8_t* dst = a.out + ((k0 / kTileK) * LDS_ROWS + row) * 64 + (unit_off % 64);
            if constexpr (P == 16)
                *(uint2*)dst = make_uint2(image_word(f), image_word(f + 8));
            else
                *(uint32_t*)dst = image_word(f);
        } else {
            int8_t q[P];
#pragma unroll
            for (int e = 0; e < P; ++e) q[e] = (int8_t)(f[e] & 0xFFu);
            if constexpr (MODE == OUT_NK) {
#pragma unroll
                for (int c = 0; c < P / 8; ++c) {
                    uint32_t wd = 0;
#pragma unroll
                    for (int u2 = 0; u2 < 4; ++u2)
                        wd |= (nib(q[8 * c + 2 * u2]) | (nib(q[8 * c + 2 * u2 + 1]) << 4)) << (8 * u2);
                    *(uint32_t*)(a.out + row * (a.K / 2) + (k0 + 8 * c) / 2) = wd;
                }
            } else {  // OUT_ROWMAJOR
#pragma unroll
                for (int c = 0; c < P / 8; ++c)
                    *(uint2*)(a.out + row * a.K + k0 + 8 * c) = make_uint2(pack4_i8(q + 8 * c), pack4_i8(q + 8 * c + 4));
                if (a.rotated) {
#pragma unroll
                    for (int e = 0; e < P; e += 4)
                        *(float4*)(a.rotated + row * a.K + k0 + e) = make_float4(r[e], r[e + 1], r[e + 2], r[e + 3]);
                }
            }
        }
    }
}

// Occupancy targets: the largest number of waves per SIMD at which the
// instance keeps every value in registers (a spill costs more than the lost
// wave: g = 256 runs 1.1 us faster on 1536 x 3072 at 5 waves than at 6).
template <int G, bool REG>
constexpr int kPrepWavesPerSimd = G == 256 ? (REG ? 4 : 5) : (REG ? 5 : 6);

template <int G, int MODE, bool REG>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(kPrepWavesPerSimd<G, REG>))) void prep_kernel(
    PrepArgs a)
{
    using S = PrepShape<G>;
    constexpr int P = S::P;
    extern __shared__ __attribute__((aligned(16))) uint8_t prep_lds[];
    __shared__ uint32_t red[2][16];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    if (a.zero && blockIdx.x == 0)  // split-K counters of the GEMM that consumes this workspace
        for (int i = tid; i < a.zero_count; i += blockDim.x) a.zero[i] = 0;
    // Rows are walked with a stride of one grid's worth of rows; the loads of
    // a lane's next row are issued before the current row is processed, into
    // the other of two register buffers (no copy between them, so the wait
    // for one row never drains the next row's loads).
    // The trip count is the same for every lane of the workgroup (rows past
    // the end are processed as empty rows and not written), so the loop is
    // uniform control flow.
    int64_t row, row_step, first;
    int t;  // lane within the row's team
    if (a.team <= 64) {
        const int per_block = blockDim.x / a.team;
        first = (int64_t)blockIdx.x * per_block;
        row = first + tid / a.team;
        row_step = (int64_t)gridDim.x * per_block;
        t = tid % a.team;
    } else {
        first = row = blockIdx.x;
        row_step = gridDim.x;
        t = tid;
    }
    const int64_t n_it = first < a.rows_pad ? (a.rows_pad - first + row_step - 1) / row_step : 0;
    const int64_t k0 = (int64_t)t * P;  // first element of the phase-1 run
    double* ld = (double*)(prep_lds + wave * S::kWaveLdsBytes);
    uint4 wa[P / 8], wb[P / 8];
    load_run<P>(a.X, row, a.ld, k0, row < a.rows, wa);
    for (int64_t it = 0; it < n_it; it += 2) {
        int64_t nx = row + row_step;
        load_run<P>(a.X, nx, a.ld, k0, nx < a.rows, wb);
        prep_row<G, MODE, 0, REG>(a, wa, row, t, k0, lane, wave, ld, red, 0, 0, blockDim.x >> 6);
        row = nx;
        if (it + 1 >= n_it) break;
        nx = row + row_step;
        load_run<P>(a.X, nx, a.ld, k0, nx < a.rows, wa);
        prep_row<G, MODE, 0, REG>(a, wb, row, t, k0, lane, wave, ld, red, 1, 0, blockDim.x >> 6);
        row = nx;
    }
}

// ---------------------------------------------------------------------------
// prep_team_kernel: the operand-image mode of prep_kernel for rows whose team
// is whole waves (K_pad / P = 128 .. 1024 lanes: K_pad >= 2048 at g = 256,
// >= 1024 at g = 64) -- the activations of every FLUX-shaped linear and the
// rows of every weight.  One workgroup is one row's team and walks rows with
// a grid stride, so the row index and every row base address are uniform
// (scalar registers); the lanes only add 32-bit offsets.  The rotation is
// prep_row's (the same binary64 butterflies and LDS transposes, the same
// single rounding); the quantizer rounds the exact product r * rcp(s) with a
// fused multiply-add and keeps prep_row's near-tie fallback to the IEEE
// division; the FP6 fields reuse the rounded codes.  OUT4 / OUT6: write the
// INT4 image / the FP6 image (a linear whose plan reads only one of them
// writes only that one).  ONE_ROW: the grid has a workgroup for every row
// (launched so when the resident grid covers all rows), so there is no row
// loop at all.
// ---------------------------------------------------------------------------

// clamp(rint(fl32(r / s)), -7, 7) for P values, as the bit patterns f of
// 1.5 * 2^23 + code (low byte = the code) and as floats t.  fma(r, inv,
// 1.5 * 2^23) rounds the exact product r * inv to an integer (the sum lies in
// [2^23, 2^24), whose spacing is 1; ties to even), and fma(r, inv, -t) is that
// product's distance to the integer, rounded once.  With inv = rcp(s) (one
// ulp), r * inv is within 2^-20 of r / s and fl32(r / s) within 2^-21 of it
// (|r / s| < 8); so when the distance is at most 0.5 - 2^-18 the integer is
// rint(fl32(r / s)).  Otherwise -- and for a scale that is not a normal
// number -- the element takes the correctly rounded division.
template <int P>
__device__ inline void quantize_fma(const float (&r)[P], float s, bool zero_row, uint32_t (&f)[P], float (&t)[P])
{
    constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
    const bool exact_only = !(s >= 0x1p-126f);
    const float inv = exact_only ? 0.0f : __builtin_amdgcn_rcpf(s);
    float dmax = 0.0f;  // the largest distance to the rounded value (one compare for all P)
#pragma unroll
    for (int e = 0; e < P; ++e) {
        const float fy = __builtin_fmaf(r[e], inv, kMagic);
        t[e] = fy - kMagic;
        dmax = fmaxf(dmax, fabsf(__builtin_fmaf(r[e], inv, -t[e])));
        f[e] = __float_as_uint(fy);
    }
    const bool need = exact_only || dmax > 0.5f - 0x1p-18f;
    if (need && !zero_row) {
#pragma unroll
        for (int e = 0; e < P; ++e) {
            const float fy = __builtin_fmaf(r[e], inv, kMagic);
            const float te = fy - kMagic;
            if (exact_only || fabsf(__builtin_fmaf(r[e], inv, -te)) > 0.5f - 0x1p-18f) {
                const float q = __builtin_rintf(fminf(fmaxf(r[e] / s, -7.0f), 7.0f));  // IEEE division
                f[e] = __float_as_uint(q + kMagic);
                t[e] = __uint_as_float(f[e]) - kMagic;  // +0 for a zero code (rint may give -0)
            }
        }
    }
    if (zero_row) {
#pragma unroll
        for (int e = 0; e < P; ++e) {
            f[e] = __float_as_uint(kMagic);
            t[e] = 0.0f;
        }
    }
}

// FP6 fields of P = 8 or 16 codes given as floats (see fp6_fields)
template <int P>
__device__ inline u32x6_t fp6_fields_of(const float (&t)[P])
{
    f32x16_t ev = __builtin_nondeterministic_value(ev), od = __builtin_nondeterministic_value(od);
#pragma unroll
    for (int i = 0; i < P / 2; ++i) {
        ev[i] = t[2 * i];
        od[i] = t[2 * i + 1];
    }
    return __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(ev, od, 1.0f);
}

// The lane's P bf16 values of row `row` (uniform), k0 .. k0 + P - 1, in
// 16-byte chunks; chunks past the row's ld values or past its rows read the
// row's first chunk (a valid address) and are zeroed by team_zero_unless.
template <int P>
__device__ inline void team_load(const PrepArgs& a, int64_t row, uint32_t k0, uint4 (&w)[P / 8])
{
    const bool has_row = row < a.rows;
    const uint16_t* xr = a.X + (has_row ? row : 0) * a.ld;
#pragma unroll
    for (int c = 0; c < P / 8; ++c) {
        const uint32_t k = k0 + 8 * c;
        const uint16_t* src = xr + (has_row && k < (uint32_t)a.ld ? k : 0u);
        if (a.x_stream) {
            const v4i v = __builtin_nontemporal_load((const v4i*)src);
            w[c] = make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
        } else {
            w[c] = *(const uint4*)src;
        }
    }
}

template <int P>
__device__ inline void team_zero_unless(const PrepArgs& a, int64_t row, uint32_t k0, uint4 (&w)[P / 8])
{
    const bool has_row = row < a.rows;
#pragma unroll
    for (int c = 0; c < P / 8; ++c)
        if (!(has_row && k0 + 8 * c < (uint32_t)a.ld)) w[c] = make_uint4(0, 0, 0, 0);
}

template <int G, bool REG, bool OUT4, bool OUT6>
__device__ __forceinline__ void team_row(const PrepArgs& a, uint4 (&w)[PrepShape<G>::P / 8], int64_t row, uint32_t k0,
                                         uint32_t off4, uint32_t off6, int lane, int wave, int nw, double* ld,
                                         uint32_t (*red)[16], int parity)
{
    using S = PrepShape<G>;
    constexpr int P = S::P;
    const int gbase = (lane / P) * P;
    const int lo = lane % P;
    float* lf = (float*)ld;
    // a row of data whose every lane holds input values needs no zeroing
    // (uniform test: rows of the FLUX shapes skip it)
    if (!(row < a.rows && a.ld == a.K_pad && (int64_t)blockDim.x * P == a.K_pad)) team_zero_unless<P>(a, row, k0, w);
    // ---- phase 1: P consecutive elements, butterflies over the low bits ----
    double v[P];
#pragma unroll
    for (int c = 0; c < P / 8; ++c) {
        v[8 * c + 0] = bf16_lo(w[c].x); v[8 * c + 1] = bf16_hi(w[c].x);
        v[8 * c + 2] = bf16_lo(w[c].y); v[8 * c + 3] = bf16_hi(w[c].y);
        v[8 * c + 4] = bf16_lo(w[c].z); v[8 * c + 5] = bf16_hi(w[c].z);
        v[8 * c + 6] = bf16_lo(w[c].w); v[8 * c + 7] = bf16_hi(w[c].w);
    }
    if constexpr (REG) regular_input_signs<G, P>((int64_t)k0, v);
#pragma unroll
    for (int b = 1; b < P; b <<= 1)
#pragma unroll
        for (int e = 0; e < P; ++e)
            if (!(e & b)) {
                const double x = v[e], y = v[e | b];
                v[e] = x + y;
                v[e | b] = x - y;
            }
    // ---- transpose through this wave's LDS region, half a group at a time ----
    double u[P];
    {
        const int slot_base = (lane / P) * (P / 2);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            if (lo / (P / 2) == hh) {
                double* dst = ld + (slot_base + lo % (P / 2)) * S::kRunD;
#pragma unroll
                for (int e = 0; e < P; e += 2) *(double2*)(dst + e) = make_double2(v[e], v[e + 1]);
            }
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
#pragma unroll
            for (int i = 0; i < P / 2; ++i) u[hh * (P / 2) + i] = ld[(slot_base + i) * S::kRunD + lo];
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_s_waitcnt(0xC07F);  // every lane's reads are done before the region is rewritten
            __builtin_amdgcn_wave_barrier();
        }
    }
    // ---- phase 2: butterflies over the high bits ----
#pragma unroll
    for (int b = 1; b < P; b <<= 1)
#pragma unroll
        for (int i = 0; i < P; ++i)
            if (!(i & b)) {
                const double x = u[i], y = u[i | b];
                u[i] = x + y;
                u[i | b] = x - y;
            }
    // ---- round once to binary32, back to phase-1 order through LDS ----
    constexpr double kNorm = (G == 256) ? 0.0625 : 0.125;  // 1/sqrt(g), exact
#pragma unroll
    for (int i = 0; i < P; ++i) lf[(gbase + i) * S::kRunF + lo] = (float)(u[i] * kNorm);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0xC07F);
    float r[P];
    if constexpr (!REG) {
#pragma unroll
        for (int e = 0; e < P; e += 4) {
            const float4 q = *(const float4*)(lf + lane * S::kRunF + e);
            r[e] = q.x; r[e + 1] = q.y; r[e + 2] = q.z; r[e + 3] = q.w;
        }
    } else {
        regular_output_permutation<G, P, S::kRunF>(lf, gbase, (int64_t)k0, r);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0xC07F);  // reads done before the next row rewrites the region
    __builtin_amdgcn_wave_barrier();
    // ---- row absmax: the wave, then the team's waves through LDS ----
    float lane_max = 0.0f;
#pragma unroll
    for (int e = 0; e < P; ++e) lane_max = fmaxf(lane_max, fabsf(r[e]));
    uint32_t amax_bits = team_max(__float_as_uint(lane_max), 64);
    if (lane == 0) red[parity][wave] = amax_bits;  // rewritten two rows later, after the next row's barrier
    __syncthreads();
    amax_bits = red[parity][0];
    for (int wv = 1; wv < nw; ++wv) amax_bits = max(amax_bits, red[parity][wv]);
    const float amax = __uint_as_float(amax_bits);
    const bool zero_row = !(amax > 0.0f);
    const float s = zero_row ? 0.0f : amax / 7.0f;  // IEEE binary32 division
    if (row < a.rows && k0 == 0) a.scales[row] = s;
    if (k0 >= (uint32_t)a.K_pad) return;
    uint32_t f[P];
    float t[P];
    quantize_fma<P>(r, s, zero_row, f, t);
    const int64_t rt = row >> 5;
    const int rr = (int)(row & 31);
    const int64_t KB = a.K_pad / kTileK;
    if constexpr (OUT4) {
        uint8_t* dst = a.out + (size_t)(rt * KB) * kUnitBytes + rr * 64 + (off4 ^ (row_swizzle(rr) << 4));
        if constexpr (P == 16)
            *(uint2*)dst = make_uint2(image_word(f), image_word(f + 8));
        else
            *(uint32_t*)dst = image_word(f);
    }
    if constexpr (OUT6) {
        const u32x6_t fp = fp6_fields_of<P>(t);
        uint8_t* base6 = a.out6 + (size_t)(rt * KB) * kUnit6Bytes + rr * kRow6Bytes;
        // off6 holds the K-block part (kb * 3072) in its high bits and the block
        // b and in-block byte in its low byte: block b goes to b ^ row_swizzle6
        const uint32_t blk = (off6 >> 5) & 3, inb = off6 & 31, kbo = off6 >> 7;
        uint8_t* dst = base6 + kbo + ((blk ^ (uint32_t)row_swizzle6(rr)) * 24 + inb);
        if constexpr (P == 16) {
            *(uint3*)dst = make_uint3(fp[0], fp[1], fp[2]);
        } else {
            const uint16_t hw[3] = {(uint16_t)fp[0], (uint16_t)(fp[0] >> 16), (uint16_t)fp[1]};
#pragma unroll
            for (int d = 0; d < 3; ++d) *(uint16_t*)(dst + 2 * d) = hw[d];
        }
    }
}

// Occupancy target of the team kernel: six waves per SIMD (every instance
// stays within 80 VGPRs without spilling, 55-78 in practice), so that two
// 12-wave workgroups of a 12288-value row fit on a CU.  Against the
// previous loop, which prefetched the next row into a second register
// buffer at 85-100 VGPRs and five waves: down-projection rows (12288 values)
// 22.2 -> 19.6 us, the 4096-row stress shape 15.0 -> 13.8 us.
template <int G, bool REG, bool BOTH, bool ONE_ROW>
constexpr int kPrepTeamWavesPerSimd = 6;

template <int G, bool REG, bool OUT4, bool OUT6, bool ONE_ROW>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(kPrepTeamWavesPerSimd<G, REG, OUT4 && OUT6, ONE_ROW>))) void
prep_team_kernel(PrepArgs a)
{
    using S = PrepShape<G>;
    constexpr int P = S::P;
    extern __shared__ __attribute__((aligned(16))) uint8_t prep_lds[];
    __shared__ uint32_t red[2][16];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nw = (int)(blockDim.x >> 6);
    if (a.zero && blockIdx.x == 0)  // split-K counters and status word of the GEMM that consumes this workspace
        for (int i = tid; i < a.zero_count; i += blockDim.x) a.zero[i] = 0;
    // lane parts of the image offsets (32-bit; the row parts are uniform)
    const uint32_t k0 = (uint32_t)tid * P;
    const uint32_t kb = k0 / kTileK, kl = k0 % kTileK;
    const uint32_t ks = kl / 32, h = (kl % 32) / 16, d = (kl % 16) / 8;
    // INT4: unit kb, logical chunk 2 (ks / 2) + h (swizzled by the row at the
    // store), 8-byte half ks % 2, dword d
    const uint32_t off4 = kb * kUnitBytes + ((2 * (ks / 2) + h) << 4) + (ks % 2) * 8 + d * 4;
    // FP6: unit kb, block ks (swizzled at the store), in-block byte 6 P / 8 (kl % 32 / P)
    const uint32_t off6 = (kb * kUnit6Bytes) << 7 | (ks << 5) | ((6 * P / 8) * ((kl % 32) / P));
    double* ld = (double*)(prep_lds + wave * S::kWaveLdsBytes);
    if constexpr (ONE_ROW) {
        // every row has a workgroup of its own: no next row to prefetch
        const int64_t row = blockIdx.x;
        uint4 w[P / 8];
        team_load<P>(a, row, k0, w);
        team_row<G, REG, OUT4, OUT6>(a, w, row, k0, off4, off6, lane, wave, nw, ld, red, 0);
        return;
    }
    // rows with a stride of the grid; a row's load is not overlapped with the
    // previous row inside the workgroup (a prefetch buffer cost 25-35 VGPRs
    // and halved the workgroups per CU): other workgroups on the CU fill the
    // wait
    int parity = 0;
    for (int64_t row = blockIdx.x; row < a.rows_pad; row += gridDim.x) {
        uint4 w[P / 8];
        team_load<P>(a, row, k0, w);
        team_row<G, REG, OUT4, OUT6>(a, w, row, k0, off4, off6, lane, wave, nw, ld, red, parity);
        parity ^= 1;
    }
}

// ---------------------------------------------------------------------------
// gemm_kernel
//
// The INT8 block-tile shapes (GemmShape, chosen per problem by gemm_plan):
//   shape 0: 192 (M) x 384 (N), eight waves (two per SIMD) in a 2 x 4 grid,
//            each owning 96 x 96 = 3 x 3 MFMA tiles -- the shape that covers
//            1536 x 12288 in exactly 256 tiles (the FP6 tile of 256 x 256
//            would need two rounds);
//   shape 1: 192 (M) x 192 (N), four waves (one per SIMD) in a 2 x 2 grid,
//            each owning 96 x 96 -- 1536 x 3072 in 128 tiles, two K splits
//            each, with half the partial-tile bytes of larger tiles.
// K advances 128 at a time through a ring of four LDS stages, each holding
// the tile's activation units and then its weight units of the operand image
// (2 KB each).  The image is stored in exactly the LDS order, so every
// global -> LDS copy is a straight 1 KB run per wave instruction
// (global_load_lds_dwordx4, 16 bytes per lane, no registers involved); copies
// run three stages ahead of the MFMAs.  The MFMA 32x32x32 tiles are computed
// as W . X^T, so that each lane ends up holding four consecutive output
// columns of one row.  Both operands are widened from INT4 to INT8 x 16 in
// registers right after the LDS read; the int32 sums are therefore 256 times
// the dot products and are divided by 256 (exactly) in the epilogue.
// |dot| <= 49 K <= 802816, so 256 |dot| < 2^31.
// ---------------------------------------------------------------------------

template <int SHAPE>
struct GemmShape;
template <>
struct GemmShape<0> {
    static constexpr int NW = 8, NWM = 2, BI = 3, BJ = 3;
};
template <>
struct GemmShape<1> {
    static constexpr int NW = 4, NWM = 2, BI = 3, BJ = 3;
};
constexpr int kStages = 4;
template <int SHAPE_>
struct GemmGeom : GemmShape<SHAPE_> {
    static constexpr int SHAPE = SHAPE_;
    using S = GemmShape<SHAPE>;
    static constexpr int NWN = S::NW / S::NWM;          // waves along N
    static constexpr int BM = S::NWM * 32 * S::BI;      // block tile rows
    static constexpr int BN = NWN * 32 * S::BJ;         // block tile columns
    static constexpr int WN = 32 * S::BJ;               // wave tile columns
    static constexpr int UA = BM / 32, UB = BN / 32;    // activation / weight units per stage
    static constexpr int kStageA = UA * kUnitBytes;     // activation part of a stage
    static constexpr int kStage = (UA + UB) * kUnitBytes;
    static constexpr int COPIES = (2 * (UA + UB) + S::NW - 1) / S::NW;  // 1 KB copies per wave per stage
    static constexpr int kLdsBytes = kStages * kStage;
    static_assert(BM == gemm_tile_m(SHAPE) && BN == gemm_tile_n(SHAPE), "host plan and kernel agree");
    static_assert(S::NW * 64 == gemm_threads(SHAPE) && kLdsBytes == gemm_ring_bytes(SHAPE), "host geometry agrees");
};

// Global -> LDS copy of 16 bytes per lane from base + voff (voff per lane):
// lane l's bytes land at LDS address M0 + 16 l.  Written as inline asm so
// that the compiler neither tracks the copy (and waits for it before
// unrelated LDS reads) nor needs registers for it: nothing is returned, the
// address registers are consumed at issue, and the LDS side is ordered by the
// explicit vmcnt waits of wait_copies_and_barrier.
__device__ inline void lds_copy16(const uint8_t* base, uint32_t voff, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(base), "s"(lds_addr)
                 : "memory", "m0");
}

// Wait until at most IN_FLIGHT stages of copies (COPIES each per wave) are
// outstanding, then synchronise the workgroup.  No fence: the only memory
// traffic to order is LDS (every read of a released stage has returned into
// registers) and the copies (ordered by vmcnt).  The count is a compile-time
// constant, so that the main loop body has no branches.
template <int COPIES, int IN_FLIGHT>
__device__ inline void wait_copies_and_barrier()
{
    static_assert(IN_FLIGHT >= 0 && IN_FLIGHT * COPIES <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"i"(IN_FLIGHT * COPIES) : "memory");
}

// The same with a run-time count of 0 .. kStages - 1 stages (prologue).
template <int COPIES>
__device__ inline void wait_copies_and_barrier(int stages_in_flight)
{
    if (stages_in_flight <= 0)
        wait_copies_and_barrier<COPIES, 0>();
    else if (stages_in_flight == 1)
        wait_copies_and_barrier<COPIES, 1>();
    else if (stages_in_flight == 2)
        wait_copies_and_barrier<COPIES, 2>();
    else
        wait_copies_and_barrier<COPIES, 3>();
}

// A stage is UA activation and UB weight units, two 1 KB runs each: copy c
// of 2 (UA + UB) is half c % 2 of unit c / 2, activation units first.  Wave w
// issues copies (w * COPIES + i) mod 2 (UA + UB), i < COPIES; when the copies
// do not divide evenly, the last wave's surplus copies repeat copies of the
// first wave (the same bytes to the same place), so that every wave issues
// the same number and waits for the same count.  The global addresses of a
// wave's copies differ only by the stage's K block, so their bases are
// computed once (uniform, in scalar registers).  Units past the end of the
// matrix are re-read from the last valid unit (their products land in rows /
// columns that are never stored).
template <int SHAPE>
struct StageCopies {
    const uint8_t* src[GemmGeom<SHAPE>::COPIES];  // unit row tile, half; K block 0
    uint32_t dst[GemmGeom<SHAPE>::COPIES];        // offset within a stage
};

template <int SHAPE>
__device__ inline StageCopies<SHAPE> stage_copies(const GemmArgs& a, int mt0, int nt0, int wave)
{
    using G = GemmGeom<SHAPE>;
    constexpr int TC = 2 * (G::UA + G::UB);
    StageCopies<SHAPE> sc;
#pragma unroll
    for (int i = 0; i < G::COPIES; ++i) {
        const int c = (wave * G::COPIES + i) % TC;
        const int unit = c >> 1, half = c & 1;
        const bool is_a = unit < G::UA;
        const int ua = is_a ? unit : unit - G::UA;
        const int row_tile = is_a ? min(mt0 + ua, a.MT - 1) : min(nt0 + ua, a.NT - 1);
        sc.src[i] = (is_a ? a.act : a.wgt) + (size_t)row_tile * a.KB * kUnitBytes + half * 1024;
        sc.dst[i] = (is_a ? 0 : G::kStageA) + ua * kUnitBytes + half * 1024;
    }
    return sc;
}

template <int SHAPE>
__device__ inline void issue_stage(const StageCopies<SHAPE>& sc, uint32_t stage, int kb, int lane)
{
    const uint32_t voff = (uint32_t)kb * kUnitBytes + lane * 16;
#pragma unroll
    for (int i = 0; i < GemmGeom<SHAPE>::COPIES; ++i) lds_copy16(sc.src[i], voff, stage + sc.dst[i]);
}

// INT4 codes of one 8-byte group -> 16 INT8 values x 16 in natural order
__device__ inline v4i widen_lo_hi(uint32_t w0, uint32_t w1)
{
    v4i r;
    r[0] = (int)((w0 << 4) & 0xF0F0F0F0u);
    r[1] = (int)(w0 & 0xF0F0F0F0u);
    r[2] = (int)((w1 << 4) & 0xF0F0F0F0u);
    r[3] = (int)(w1 & 0xF0F0F0F0u);
    return r;
}

// Per-lane LDS offsets of a 32*BI (M) x 32*BJ (N) wave tile: this lane's row
// of activation unit wm*BI and of weight unit wn*BJ within a stage.
struct Frag {
    int sa, sb, swz, h;
};

// Quads of one pair of k-steps: BI activation quads and BJ weight quads, each
// 16 bytes = 2 k-steps x 16 codes of this lane's row.
template <int BI, int BJ>
__device__ inline void load_pair(const Frag& f, const uint8_t* stage, int pr, uint4 (&aq)[BI], uint4 (&bq)[BJ])
{
    const int off = ((2 * pr + f.h) ^ f.swz) * 16;
#pragma unroll
    for (int i = 0; i < BI; ++i) aq[i] = *(const uint4*)(stage + f.sa + i * kUnitBytes + off);
#pragma unroll
    for (int j = 0; j < BJ; ++j) bq[j] = *(const uint4*)(stage + f.sb + j * kUnitBytes + off);
}

// Widened operands of one k-step: BI activation and BJ weight fragments of 16
// INT8 values x 16 each.
template <int BI, int BJ>
struct Wide {
    v4i a[BI], b[BJ];
};

// k-step kk (0 or 1) of a pair of quads -> widened fragments
template <int BI, int BJ>
__device__ inline void widen(const uint4 (&aq)[BI], const uint4 (&bq)[BJ], int kk, Wide<BI, BJ>& w)
{
#pragma unroll
    for (int i = 0; i < BI; ++i) w.a[i] = kk == 0 ? widen_lo_hi(aq[i].x, aq[i].y) : widen_lo_hi(aq[i].z, aq[i].w);
#pragma unroll
    for (int j = 0; j < BJ; ++j) w.b[j] = kk == 0 ? widen_lo_hi(bq[j].x, bq[j].y) : widen_lo_hi(bq[j].z, bq[j].w);
}

// acc[j][i] += W_j . X_i^T for one k-step
template <int BI, int BJ>
__device__ inline void mfmas(const Wide<BI, BJ>& w, v16i (&acc)[BJ][BI])
{
#pragma unroll
    for (int j = 0; j < BJ; ++j)
#pragma unroll
        for (int i = 0; i < BI; ++i)
            acc[j][i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(w.b[j], w.a[i], acc[j][i], 0, 0, 0);
}

// Instruction-mix hints for one k-step phase of NM MFMAs (sched_group_barrier
// masks: 0x008 MFMA, 0x100 LDS read, 0x002 VALU): each MFMA is followed by NV
// of the widening instructions of the next k-step and, where there are any,
// one LDS read, so the matrix core, the vector ALU and the LDS work side by
// side instead of in bursts.
template <int NM, int NV>
__device__ inline void interleave_mfma_valu(int lds_reads)
{
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (m < lds_reads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
    }
}

// ---------------------------------------------------------------------------
// Helpers of the split-K exchange (split_k_finish, after the epilogue).
// ---------------------------------------------------------------------------

// lds_copy16 with a device-coherent global read
__device__ inline void lds_copy16_coherent(const uint8_t* g, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off sc1"
                 :
                 : "v"(g), "s"(lds_addr)
                 : "memory", "m0");
}

// The accumulators of the two matrix-core paths: the INT8 path enters both
// operands times 16, so its int32 sums are 256 times the dot products; the
// FP6 path's binary32 sums are the dot products themselves (exact integers).
typedef float v16f __attribute__((ext_vector_type(16)));
template <typename ACC>
struct AccOps;
template <>
struct AccOps<v16i> {
    __device__ static float value(const v16i& a, int r) { return (float)(a[r] >> 8); }
    __device__ static int32_t ivalue(const v16i& a, int r) { return a[r] >> 8; }
    __device__ static uint32_t bits(const v16i& a, int r) { return (uint32_t)a[r]; }
    __device__ static void add(v16i& a, int r, uint32_t w) { a[r] += (int32_t)w; }
};
template <>
struct AccOps<v16f> {
    __device__ static float value(const v16f& a, int r) { return a[r]; }
    __device__ static int32_t ivalue(const v16f& a, int r) { return (int32_t)a[r]; }
    __device__ static uint32_t bits(const v16f& a, int r) { return __float_as_uint(a[r]); }
    __device__ static void add(v16f& a, int r, uint32_t w) { a[r] += __uint_as_float(w); }  // exact: integers < 2^24
};


// 8 when the epilogue staging row r has its 8-byte halves exchanged, else 0
__device__ inline int half_swap(int r) { return (((r >> 3) ^ (r >> 4)) & 1) * 8; }

template <int V>
struct Const {
    static constexpr int value = V;
};

// The block's epilogue parameters go straight from memory into a small LDS
// array of their own, requested before the first stage's copies, so that the
// epilogue starts without a round trip to memory: BN column scales (binary32),
// BN biases (bf16 in the low half of a 4-byte slot), BM row scales
// (binary32).  Like the stage copies they are global -> LDS DMA written as
// inline asm (nothing returned, so the compiler does not wait for them); lane
// l's element lands at M0 + 4 l, and the prologue's wait for the first stage
// also covers these older requests.  Indices are clamped and a missing bias
// reads another valid address.
template <typename G>
struct EpilogueParams {
    static constexpr int kColChunks = G::BN / 64, kRowChunks = G::BM / 64;
    static constexpr int kChunks = 2 * kColChunks + kRowChunks;  // 64 slots each
    static constexpr int kCount = 64 * kChunks;
    static_assert(G::BN % 64 == 0 && G::BM % 64 == 0, "whole 64-slot chunks");
};

__device__ inline void lds_copy4(const void* base, uint32_t voff, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                 :
                 : "v"(voff), "s"(base), "s"(lds_addr)
                 : "memory", "m0");
}

__device__ inline void lds_copy2(const void* base, uint32_t voff, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_ushort %0, %1"
                 :
                 : "v"(voff), "s"(base), "s"(lds_addr)
                 : "memory", "m0");
}

template <typename G>
__device__ inline void issue_epilogue_params(const GemmArgs& a, int tm, int tn, int wave, int lane, uint32_t params_lds)
{
    using E = EpilogueParams<G>;
    const void* bsrc = a.bias ? (const void*)a.bias : (const void*)a.sw;  // a valid address either way
    for (int c = wave; c < E::kChunks; c += G::NW) {  // uniform per wave
        const uint32_t dst = params_lds + c * 256;
        if (c < E::kColChunks) {
            const int64_t n = min((int64_t)tn * G::BN + c * 64 + lane, a.N - 1);
            lds_copy4(a.sw, (uint32_t)n * 4, dst);
        } else if (c < 2 * E::kColChunks) {
            const int64_t n = min((int64_t)tn * G::BN + (c - E::kColChunks) * 64 + lane, a.N - 1);
            lds_copy2(bsrc, (uint32_t)n * 2, dst);
        } else {
            const int64_t m = min((int64_t)tm * G::BM + (c - 2 * E::kColChunks) * 64 + lane, a.M - 1);
            lds_copy4(a.sx, (uint32_t)m * 4, dst);
        }
    }
}

// Epilogue of a block tile: int32 stores (parity hook) or scale + bias to bf16
// through LDS (every copy has landed and every wave is past its last LDS
// read of the K loop when this runs).  MASKED: only the MFMA tiles (j, i)
// whose sub-block split_sub_of(nsub, i, j) has its bit set in `subs` (the
// sub-blocks of a split-K exchange that this workgroup finished).
template <typename G, int OUT, bool MASKED = false, typename ACC>
__device__ inline void gemm_epilogue(const GemmArgs& a, int tm, int tn, int wm, int wn, int tid, int wave, int lane,
                                     uint8_t* smem, const float* params, const ACC (&acc)[G::BJ][G::BI],
                                     uint32_t subs = ~0u, int nsub = 1)
{
    constexpr int NW = G::NW, BI = G::BI, BJ = G::BJ, WN = G::WN;
    const int r32 = lane & 31, h = lane >> 5;
    auto member = [&](int j, int i) __attribute__((always_inline)) {
        return !MASKED || ((subs >> split_sub_of(G::SHAPE, nsub, i, j)) & 1u) != 0;
    };
    const int64_t m_base = (int64_t)tm * G::BM + wm * (32 * BI);
    const int64_t n_base = (int64_t)tn * G::BN + wn * WN;

    // D[row][col] of a 32x32 MFMA tile sits in lane col + 32 * ((row / 4) % 2),
    // register (row / 8) * 4 + row % 4; here rows are output columns n and
    // columns are output rows m, so lane l holds row m = l % 32 and, per group
    // of four registers t, the four consecutive columns n = 8 t + 4 h + (0..3).
    if constexpr (OUT == GEMM_OUT_I32) {
        const bool vec_ok = (a.N % 4) == 0;
#pragma unroll
        for (int i = 0; i < BI; ++i) {
            const int64_t m = m_base + 32 * i + r32;
            if (m >= a.M) continue;
#pragma unroll
            for (int j = 0; j < BJ; ++j) {
                if (!member(j, i)) continue;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int64_t n0 = n_base + 32 * j + 8 * t + 4 * h;
                    if (n0 >= a.N) continue;
                    int32_t v[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) v[u] = AccOps<ACC>::ivalue(acc[j][i], 4 * t + u);
                    int32_t* dst = (int32_t*)a.out + m * a.N + n0;
                    if (vec_ok) {
                        *(int4*)dst = make_int4(v[0], v[1], v[2], v[3]);
                    } else {
                        for (int u = 0; u < 4 && n0 + u < a.N; ++u) dst[u] = v[u];
                    }
                }
            }
        }
    } else {
        // The block's column scales, biases and row scales are in params
        // (parked there before the K loop).  The bf16 output goes through a
        // per-wave LDS tile of 32 rows x WN columns, one MFMA tile row at a
        // time, and is stored as 16-byte row segments.  Row pitch 2*WN + 16
        // bytes (36 banks modulo 64) keeps rows 16-byte aligned; rows r and
        // r + 16 would still meet on the same banks, so in rows with
        // half_swap(r) the two 8-byte halves of every 16-byte chunk trade
        // places: the 8-byte writes of 16 (32-bank LDS) or 32 (64-bank LDS)
        // consecutive lanes then hit distinct banks.
        const float* p_sw = params;
        const uint32_t* p_b = (const uint32_t*)params + G::BN;  // bf16 in the low half
        const float* p_sx = params + 2 * G::BN;
        const bool has_bias = a.bias != nullptr;
        constexpr int kPitch = 2 * WN + 16;
        constexpr int kChunks = WN / 8;              // 16-byte chunks per tile row
        constexpr int kReads = 32 * kChunks / 64;    // chunks per lane per tile row block
        static_assert(kReads * 64 == 32 * kChunks, "row chunks divide evenly over the lanes");
        static_assert(NW * 32 * kPitch <= G::kLdsBytes, "epilogue staging must fit in LDS");
        __syncthreads();  // every wave is past its last read of the ring; params are visible
        uint8_t* tile_lds = smem + wave * (32 * kPitch);
        const bool vec8 = (a.N % 8) == 0;
#pragma unroll
        for (int i = 0; i < BI; ++i) {
            bool any = false;
#pragma unroll
            for (int j = 0; j < BJ; ++j) any = any || member(j, i);
            if (!any) continue;
            const float sxm = p_sx[wm * (32 * BI) + 32 * i + r32];
#pragma unroll
            for (int j = 0; j < BJ; ++j) {
                if (!member(j, i)) continue;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int nl = 32 * j + 8 * t + 4 * h;  // column within the wave tile
                    const float4 sw4 = *(const float4*)(p_sw + wn * WN + nl);
                    const uint4 b4 = *(const uint4*)(p_b + wn * WN + nl);
                    const float sc[4] = {sw4.x, sw4.y, sw4.z, sw4.w};
                    const float bb[4] = {has_bias ? __uint_as_float(b4.x << 16) : 0.0f,
                                         has_bias ? __uint_as_float(b4.y << 16) : 0.0f,
                                         has_bias ? __uint_as_float(b4.z << 16) : 0.0f,
                                         has_bias ? __uint_as_float(b4.w << 16) : 0.0f};
                    float y[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        y[u] = __builtin_fmaf(AccOps<ACC>::value(acc[j][i], 4 * t + u) * sxm, sc[u], bb[u]);
                    }
                    *(uint2*)(tile_lds + r32 * kPitch + ((nl * 2) ^ half_swap(r32))) =
                        make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
                }
            }
            // read back row segments: lane l takes the 16-byte chunks l + 64 s
            // of the tile row block (row rho = chunk / kChunks)
#pragma unroll
            for (int sr = 0; sr < kReads; ++sr) {
                const int idx = lane + 64 * sr;
                const int rho = idx / kChunks;
                const int c = idx % kChunks;
                if (!member(c / 4, i)) continue;  // chunk c: columns 8c .. 8c + 7, in MFMA tile j = c / 4
                uint4 w = *(const uint4*)(tile_lds + rho * kPitch + c * 16);
                if (half_swap(rho)) w = make_uint4(w.z, w.w, w.x, w.y);
                const int64_t m = m_base + 32 * i + rho;
                const int64_t n = n_base + 8 * c;
                if (m >= a.M || n >= a.N) continue;
                uint16_t* dst = (uint16_t*)a.out + m * a.N + n;
                if (vec8 && n + 8 <= a.N) {
                    // streaming store: Y is not read back by this kernel, and
                    // keeping it out of the caches shortens the final drain
                    __builtin_nontemporal_store(v4i{(int)w.x, (int)w.y, (int)w.z, (int)w.w}, (v4i*)dst);
                } else {
                    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
                    for (int u = 0; u < 8 && n + u < a.N; ++u) dst[u] = (uint16_t)(ww[u >> 1] >> (16 * (u & 1)));
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Split-K exchange, spread over the S workgroups of a split tile.  The tile's
// MFMA tiles (j, i) of every wave ("pairs") form S sub-blocks of consecutive
// pairs in row-major order (split_sub_of, layout.h).  Each workgroup visits the S
// sub-blocks in turn, starting at its own split index, and takes a ticket
// from the sub-block's counter (split_counter, layout.h).  The first S - 1
// ticket holders store their partial sums of the sub-block (4-byte words)
// into slot `ticket` of the tile (split_store_offset) with device-coherent
// stores, wait until the stores have completed and count themselves finished.
// The last ticket holder waits until S - 1 writers have finished -- each of
// them holds a ticket, so it is running, and between taking a ticket and
// counting itself finished a workgroup never waits -- then copies the
// sub-block's pairs of every slot into its LDS ring with device-coherent
// global -> LDS copies, adds them (exact integer sums, any order) and returns
// the sub-block's two counters to zero for the next launch.  One epilogue at
// the end writes the sub-blocks the workgroup finished.  The workgroups of a
// tile usually reach the
// exchange together, so with the rotated visiting order each of them
// finishes one sub-block: a workgroup stores, loads and outputs about 1/S of
// a tile instead of one workgroup loading S - 1 tiles and writing all of Y
// (a compute unit moves device-coherent data at only some 20-30 GB/s).
// The wait is bounded (a.spin_limit sleeps).  If it runs out, the finalizer
// sets the workspace's status word to kStatusSplitTimeout, adds no slot
// (their contents are not known to be written), leaves the counters as they
// are (the next activation step clears them and the status word), and still
// runs the epilogue, so the kernel ends normally and the caller can see the
// failure.  a.extra_wait makes a finalizer wait for that many writers more
// than exist (a test of this path: the wait then always runs out).
// Device-coherent (agent-scope, sc1) accesses go to the level of the memory
// system that every compute unit sees, so no cache-wide write-back or
// invalidation is needed.
// ---------------------------------------------------------------------------
template <typename G, int OUT, typename ACC>
__device__ inline void split_k_finish(const GemmArgs& a, int tile, int split, int tm, int tn, int wm, int wn, int tid,
                                      int wave, int lane, uint32_t lds0, uint8_t* smem, const float* params,
                                      ACC (&acc)[G::BJ][G::BI])
{
    constexpr int BI = G::BI, BJ = G::BJ;
    constexpr int SHAPE = G::SHAPE;
    constexpr int kThreads = G::NW * 64;
    constexpr int kPairs = BI * BJ;
    constexpr int kPairBytes = split_pair_bytes(SHAPE);
    constexpr int kPairChunks = kPairBytes / 1024 / G::NW;  // 1 KB copies per wave and pair
    constexpr int kRingPairs = split_pairs_per_copy(SHAPE);  // pairs the ring holds at once
    static_assert(kThreads == gemm_threads(SHAPE) && kPairs * 8 == split_words_per_thread(SHAPE),
                  "slot geometry of layout.h");
    static_assert(kPairChunks * 1024 * G::NW == kPairBytes && kRingPairs >= 1, "pair copies fit the ring");
    static_assert(BI == gemm_wave_tiles_m(SHAPE) && BJ == gemm_wave_tiles_n(SHAPE), "pair geometry of layout.h");
    __shared__ int ticket_sh;
    __shared__ int done_sh;
    const int S = a.splits;
    uint8_t* part = (uint8_t*)a.partial;
    uint32_t mine = 0;  // the sub-blocks this workgroup finishes
    for (int k = 0; k < S; ++k) {
        const int b = (split + k) % S;
        uint32_t* tickets = a.counters + split_counter(tile, S, b);
        uint32_t* finished = tickets + kSplitCounters;
        if (tid == 0) ticket_sh = (int)__hip_atomic_fetch_add(tickets, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();  // on the first visit also: every wave is done with the stage ring
        const int ticket = ticket_sh;
        if (ticket < S - 1) {
#pragma unroll
            for (int p = 0; p < kPairs; ++p) {
                const int j = p / BI, i = p % BI;
                if (split_sub_of(SHAPE, S, i, j) != b) continue;
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    // 8-byte word 8 p + q of this thread: registers 2q, 2q + 1
                    const uint64_t v = (uint64_t)AccOps<ACC>::bits(acc[j][i], 2 * q) |
                                       ((uint64_t)AccOps<ACC>::bits(acc[j][i], 2 * q + 1) << 32);
                    __hip_atomic_store((uint64_t*)(part + split_store_offset(SHAPE, tile, S, ticket, 8 * p + q, tid)), v,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            __builtin_amdgcn_s_waitcnt(0);  // every store of this wave has completed
            __syncthreads();
            if (tid == 0) __hip_atomic_fetch_add(finished, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            continue;
        }
        if (tid == 0) {
            // bounded: the writers are running and never wait
            const uint32_t need = (uint32_t)(S - 1 + a.extra_wait);
            int done = 0;
            for (int spin = 0; spin < a.spin_limit; ++spin) {
                if (__hip_atomic_load(finished, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= need) {
                    done = 1;
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
            if (done) {
                __hip_atomic_store(tickets, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(finished, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            } else {
                __hip_atomic_store(a.status, kStatusSplitTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            done_sh = done;
        }
        __syncthreads();
        mine |= 1u << b;
        if (done_sh) {
            // the sub-block's pairs are row-major numbers first + m,
            // m = 0 .. members - 1; the ring takes kRingPairs of them per round
            const int first = split_sub_first(SHAPE, S, b);
            const int members = split_sub_first(SHAPE, S, b + 1) - first;
            for (int sl = 0; sl < S - 1; ++sl)
                for (int m0 = 0; m0 < members; m0 += kRingPairs) {
                    const int m1 = min(members, m0 + kRingPairs);
                    for (int m = m0; m < m1; ++m)
#pragma unroll
                        for (int c = 0; c < kPairChunks; ++c) {
                            const int chunk = wave * kPairChunks + c;
                            lds_copy16_coherent(
                                part + split_copy_offset(SHAPE, tile, S, sl, split_pair_of(SHAPE, first + m), chunk, lane),
                                lds0 + (m - m0) * kPairBytes + chunk * 1024);
                        }
                    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
                    for (int p = 0; p < kPairs; ++p) {
                        const int j = p / BI, i = p % BI;
                        const int m = i * BJ + j - first;
                        if (m < m0 || m >= m1) continue;
                        const uint8_t* src = smem + (m - m0) * kPairBytes;
#pragma unroll
                        for (int q = 0; q < 8; ++q) {
                            const uint2 w = *(const uint2*)(src + ((size_t)q * kThreads + tid) * 8);
                            AccOps<ACC>::add(acc[j][i], 2 * q, w.x);
                            AccOps<ACC>::add(acc[j][i], 2 * q + 1, w.y);
                        }
                    }
                    __syncthreads();  // every read of the ring is done before the next copies
                }
        }
    }
    if (mine) gemm_epilogue<G, OUT, true>(a, tm, tn, wm, wn, tid, wave, lane, smem, params, acc, mine, S);
}

// SPLIT: the instance that takes part in a split-K exchange (launched only
// when a.splits > 1); the other instance has no exchange code at all, which
// keeps its registers free of spills.
template <int OUT, int SHAPE, bool SPLIT>
__global__ __launch_bounds__(GemmShape<SHAPE>::NW * 64, 1) void gemm_kernel(GemmArgs a)
{
    using G = GemmGeom<SHAPE>;
    constexpr int BI = G::BI, BJ = G::BJ;
    constexpr int kStage = G::kStage;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kStage];
    __shared__ __attribute__((aligned(16))) float params[EpilogueParams<G>::kCount];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps copy addresses scalar
    const int wm = wave % G::NWM, wn = wave / G::NWM;

    // XCD-aware order: workgroup i runs on XCD i % 8; give each XCD a
    // contiguous range of (split, tile) items -- splits slowest, row tiles
    // fastest -- so workgroups sharing weight columns and a K range share
    // that XCD's L2.
    const int tiles = a.tiles_m * a.tiles_n;
    const int total = tiles * a.splits;
    const int wg = blockIdx.x;
    const int qx = total / 8, rx = total % 8;
    const int xcd = wg % 8, idx = wg / 8;
    const int vid = xcd * qx + (xcd < rx ? xcd : rx) + idx;
    const int split = vid / tiles, tile = vid % tiles;
    const int tm = tile % a.tiles_m, tn = tile / a.tiles_m;
    const int mt0 = tm * G::UA, nt0 = tn * G::UB;
    // this workgroup's K blocks: [kb0, kb0 + KC)
    const int kb0 = (int)((int64_t)split * a.KB / a.splits);
    const int KC = (int)((int64_t)(split + 1) * a.KB / a.splits) - kb0;

    v16i acc[BJ][BI];
#pragma unroll
    for (int j = 0; j < BJ; ++j)
#pragma unroll
        for (int i = 0; i < BI; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[j][i][r] = 0;

    const int r32 = lane & 31, h = lane >> 5;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)smem);
    Frag f;
    f.sa = (wm * BI) * kUnitBytes + r32 * 64;
    f.sb = G::kStageA + (wn * BJ) * kUnitBytes + r32 * 64;
    f.swz = row_swizzle(r32);
    f.h = h;

    // prologue: the epilogue's parameters, then the first kStages stages in
    // flight; wait for stage 0 (and so for the older parameter copies)
    if constexpr (OUT == GEMM_OUT_BF16)
        issue_epilogue_params<G>(a, tm, tn, wave, lane,
                                 __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)params));
    const int first = KC < kStages ? KC : kStages;
    const StageCopies<SHAPE> sc = stage_copies<SHAPE>(a, mt0, nt0, wave);
    for (int s = 0; s < first; ++s) issue_stage<SHAPE>(sc, lds0 + s * kStage, kb0 + s, lane);
    wait_copies_and_barrier<G::COPIES>(first - 1);
    uint4 aq[2][BI], bq[2][BJ];
    Wide<BI, BJ> w[2];
    load_pair<BI, BJ>(f, smem, 0, aq[0], bq[0]);
    widen<BI, BJ>(aq[0], bq[0], 0, w[0]);

    // Per stage kb (buffer kb % kStages):
    //   k-step 0 MFMAs | reads of pair 1 of this stage, widening of k-step 1
    //   k-step 1 MFMAs | widening of k-step 2 (pair 1)
    //   barrier: stage kb + 1 has landed everywhere, and every wave has
    //            consumed this stage's buffer, which takes the copy of stage
    //            kb + kStages (so copies run three stages ahead)
    //   k-step 2 MFMAs | reads of pair 0 of stage kb + 1, widening of k-step 3
    //   k-step 3 MFMAs | widening of k-step 0 of stage kb + 1
    // LDS reads thus come in two even halves per stage and the barrier sits
    // between MFMA phases.  sched_barrier(0) keeps the phases in this order
    // (nothing hoisted above the barrier, no read sunk below its phase).
    constexpr int NM = BI * BJ;                  // MFMAs per k-step
    constexpr int NR = BI + BJ;                  // LDS reads per pair
    constexpr int NV = 6 * (BI + BJ) / NM + 1;   // widening instructions per MFMA
    // One stage.  ISSUE: copy stage kr + kStages into the buffer this stage
    // frees; IN_FLIGHT: stages that may still be in flight at the barrier;
    // MORE: a stage kr + 1 follows.  All three are compile-time constants, so
    // each call is straight-line code and the phase hints above hold.
    auto step = [&](int kr, auto issue_c, auto in_flight_c, auto more_c) __attribute__((always_inline)) {
        constexpr bool ISSUE = decltype(issue_c)::value != 0;
        constexpr int IN_FLIGHT = decltype(in_flight_c)::value;
        constexpr bool MORE = decltype(more_c)::value != 0;
        const int slot = kr % kStages;
        const uint8_t* cur = smem + slot * kStage;
        load_pair<BI, BJ>(f, cur, 1, aq[1], bq[1]);
        mfmas<BI, BJ>(w[0], acc);
        widen<BI, BJ>(aq[0], bq[0], 1, w[1]);
        interleave_mfma_valu<NM, NV>(NR);
        __builtin_amdgcn_sched_barrier(0);
        mfmas<BI, BJ>(w[1], acc);
        widen<BI, BJ>(aq[1], bq[1], 0, w[0]);
        interleave_mfma_valu<NM, NV>(0);
        __builtin_amdgcn_sched_barrier(0);
        wait_copies_and_barrier<G::COPIES, IN_FLIGHT>();
        if constexpr (ISSUE) issue_stage<SHAPE>(sc, lds0 + slot * kStage, kb0 + kr + kStages, lane);
        if constexpr (MORE) load_pair<BI, BJ>(f, smem + ((kr + 1) % kStages) * kStage, 0, aq[0], bq[0]);
        __builtin_amdgcn_sched_barrier(0);
        mfmas<BI, BJ>(w[0], acc);
        widen<BI, BJ>(aq[1], bq[1], 1, w[1]);
        interleave_mfma_valu<NM, NV>(MORE ? NR : 0);
        __builtin_amdgcn_sched_barrier(0);
        mfmas<BI, BJ>(w[1], acc);
        if constexpr (MORE) widen<BI, BJ>(aq[0], bq[0], 0, w[0]);
        interleave_mfma_valu<NM, NV>(0);
        __builtin_amdgcn_sched_barrier(0);
    };
    // Steady state: stage kr + 1 must have landed, stages kr + 2 and kr + 3
    // may be in flight, stage kr + 4 is issued.  Then the last four stages
    // (fewer of them when KC < 4), which copy nothing and wait for less.
    static_assert(kStages == 4, "the tail below is written for four stages");
    for (int kr = 0; kr < KC - kStages; ++kr) step(kr, Const<1>{}, Const<2>{}, Const<1>{});
    if (KC >= 4) step(KC - 4, Const<0>{}, Const<2>{}, Const<1>{});
    if (KC >= 3) step(KC - 3, Const<0>{}, Const<1>{}, Const<1>{});
    if (KC >= 2) step(KC - 2, Const<0>{}, Const<0>{}, Const<1>{});
    step(KC - 1, Const<0>{}, Const<0>{}, Const<0>{});

    if constexpr (SPLIT)
        split_k_finish<G, OUT>(a, tile, split, tm, tn, wm, wn, tid, wave, lane, lds0, smem, params, acc);
    else
        gemm_epilogue<G, OUT>(a, tm, tn, wm, wn, tid, wave, lane, smem, params, acc);
}

// ---------------------------------------------------------------------------
// gemm6_kernel: the block-tile product on the FP6 matrix cores.
//
// The codes come from the FP6 images (layout.h): every integer code in
// [-7, 7] is an exact e2m3 value, v_mfma_scale_f32_32x32x64_f8f6f4 with unit
// block scales multiplies them exactly, and the binary32 sums are the exact
// integer dot products (|dot| <= 802816 < 2^24), at twice the INT8 rate and
// with no widening in registers.
// Block tile 256 x 256 (Gemm6Geom: waves, their grid and MFMA tiles per wave).
// K advances 128 at a time through a ring of three 48 KB LDS stages filled by
// global -> LDS copies, two stages ahead.  A stage is two k-steps of 64; a lane's fragment
// for one k-step is 24 bytes (32 codes), read as three ds_read_b64:
//   k-step 0 fragments (X registers) feed 16 MFMAs while the k-step 1
//     fragments of the same stage are read into Y;
//   barrier: the next stage has landed everywhere and every wave is done
//     reading this stage, whose buffer then takes the copy three stages on;
//   Y feeds 16 MFMAs while the next stage's k-step 0 fragments are read into X
//     (the reads interleaved with the MFMAs: a wave stalls once 15 LDS reads
//     are outstanding).
// Each stage so starts and ends with the same registers, and the body is
// straight-line code.
// ---------------------------------------------------------------------------
template <int NW_, int NWM_, int BI_, int BJ_, int SHAPE_, int STAGES_ = 3>
struct Gemm6Geom {
    static constexpr int NW = NW_, NWM = NWM_, BI = BI_, BJ = BJ_, SHAPE = SHAPE_;
    static constexpr int NWN = NW / NWM;
    static constexpr int BM = NWM * 32 * BI, BN = NWN * 32 * BJ, WN = 32 * BJ;
    static constexpr int UA = BM / 32, UB = BN / 32;
    static constexpr int kStageA = UA * kUnit6Bytes;
    static constexpr int kStage = (UA + UB) * kUnit6Bytes;
    static constexpr int kStages = STAGES_;
    static constexpr int kLdsBytes = kStages * kStage;
    static constexpr int kChunks = 3 * (UA + UB);                 // 1 KB copies per stage
    static constexpr int COPIES = (kChunks + NW - 1) / NW;        // per wave (the last ones may repeat)
    static_assert(kStages == 2 || kStages == 3, "the stage loop is written for two or three stages");
    static_assert(BM == gemm_tile_m(SHAPE) && BN == gemm_tile_n(SHAPE), "host plan and kernel agree");
    static_assert(NW * 64 == gemm_threads(SHAPE) && kLdsBytes == gemm_ring_bytes(SHAPE), "host geometry agrees");
};
// Shape 2: eight waves, two per SIMD, each owning 128 x 64.  (Four waves of
// 128 x 128 read a third fewer LDS bytes per MFMA, but with one wave per SIMD
// every LDS wait stalls the matrix core: measured 14% slower on 1536 x 3072 x
// 9216, and its epilogue has twice the work per wave.)
using Gemm6W8 = Gemm6Geom<8, 2, 4, 2, 2>;
// Shape 3: 192 x 384, eight waves of 96 x 96 (3 x 3 MFMA tiles); a stage is
// 54 KB, so the ring holds two.
using Gemm6Wide = Gemm6Geom<8, 2, 3, 3, 3, 2>;

typedef int v8i __attribute__((ext_vector_type(8)));

// one lane's fragment (three 8-byte slots) as the MFMA operand: e2m3 reads
// six registers
__device__ inline v8i fp6_operand(const uint2 (&p)[3])
{
    v8i r = __builtin_nondeterministic_value(r);
    r[0] = (int)p[0].x;
    r[1] = (int)p[0].y;
    r[2] = (int)p[1].x;
    r[3] = (int)p[1].y;
    r[4] = (int)p[2].x;
    r[5] = (int)p[2].y;
    return r;
}

// Wait until at most IN_FLIGHT stages of this wave's copies are outstanding
// and its LDS reads have returned, then synchronise the workgroup.
template <int COPIES, int IN_FLIGHT>
__device__ inline void wait6_and_barrier()
{
    static_assert(IN_FLIGHT >= 0 && IN_FLIGHT * COPIES <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"i"(IN_FLIGHT * COPIES) : "memory");
}

template <int OUT, typename G, bool SPLIT>
__global__ __launch_bounds__(G::NW * 64, 1) void gemm6_kernel(GemmArgs a)
{
    constexpr int BI = G::BI, BJ = G::BJ;
    constexpr int kStage = G::kStage;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[G::kLdsBytes];
    __shared__ __attribute__((aligned(16))) float params[EpilogueParams<G>::kCount];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % G::NWM, wn = wave / G::NWM;

    // XCD-aware order, as in gemm_kernel
    const int tiles = a.tiles_m * a.tiles_n;
    const int total = tiles * a.splits;
    const int wg = blockIdx.x;
    const int qx = total / 8, rx = total % 8;
    const int xcd = wg % 8, idx = wg / 8;
    const int vid = xcd * qx + (xcd < rx ? xcd : rx) + idx;
    const int split = vid / tiles, tile = vid % tiles;
    const int tm = tile % a.tiles_m, tn = tile / a.tiles_m;
    const int kb0 = (int)((int64_t)split * a.KB / a.splits);
    const int KC = (int)((int64_t)(split + 1) * a.KB / a.splits) - kb0;

    v16f acc[BJ][BI];
#pragma unroll
    for (int j = 0; j < BJ; ++j)
#pragma unroll
        for (int i = 0; i < BI; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.0f;

    // Copies: a stage is 3 (UA + UB) runs of 1 KB (activation units 0 ..
    // UA - 1, then the weight units, three runs each); wave w moves runs
    // COPIES w .. COPIES (w + 1) - 1, and where they do not divide evenly the
    // last wave repeats the final run (same bytes to the same place), so that
    // every wave waits for the same count.  Units past the end of the matrix
    // re-read the last valid unit (their products land in rows / columns
    // that are never stored).
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)smem);
    const uint8_t* copy_src[G::COPIES];
    uint32_t copy_dst[G::COPIES];
#pragma unroll
    for (int i = 0; i < G::COPIES; ++i) {
        const int c = min(wave * G::COPIES + i, G::kChunks - 1);
        const int ug = c / 3, part = c % 3;
        const bool is_a = ug < G::UA;
        const int row_tile = is_a ? min(tm * G::UA + ug, a.MT - 1) : min(tn * G::UB + ug - G::UA, a.NT - 1);
        copy_src[i] = (is_a ? a.act6 : a.wgt6) + (size_t)row_tile * a.KB * kUnit6Bytes + part * 1024;
        copy_dst[i] = (uint32_t)(ug * kUnit6Bytes + part * 1024);
    }
    auto issue = [&](uint32_t stage, int kb) __attribute__((always_inline)) {
        const uint32_t voff = (uint32_t)kb * kUnit6Bytes + lane * 16;
#pragma unroll
        for (int i = 0; i < G::COPIES; ++i) lds_copy16(copy_src[i], voff, stage + copy_dst[i]);
    };

    // Fragments: lane (r32, h) reads row r32 of its tiles' units, block
    // 2 s + h for k-step s: three 8-byte slots at consecutive addresses.  The
    // per-tile offsets are hidden from the compiler (an empty asm), so that it
    // pairs the slots of one fragment (which land in operand order) rather
    // than the same slot of two tiles (which would need register moves).
    const int r32 = lane & 31, h = lane >> 5;
    int ta[BI], tb[BJ];
#pragma unroll
    for (int i = 0; i < BI; ++i) {
        ta[i] = (wm * BI + i) * kUnit6Bytes + r32 * kRow6Bytes;
        asm volatile("" : "+v"(ta[i]));
    }
#pragma unroll
    for (int j = 0; j < BJ; ++j) {
        tb[j] = G::kStageA + (wn * BJ + j) * kUnit6Bytes + r32 * kRow6Bytes;
        asm volatile("" : "+v"(tb[j]));
    }
    const int blk[2] = {((0 + h) ^ row_swizzle6(r32)) * 24, ((2 + h) ^ row_swizzle6(r32)) * 24};
    uint2 xa[BI][3], xb[BJ][3], ya[BI][3], yb[BJ][3];
    auto read = [&](const uint8_t* stage, int st, uint2 (&ra)[BI][3], uint2 (&rb)[BJ][3]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < BI; ++i) {
            const uint8_t* p = stage + ta[i] + blk[st];
#pragma unroll
            for (int x = 0; x < 3; ++x) ra[i][x] = *(const uint2*)(p + 8 * x);
        }
#pragma unroll
        for (int j = 0; j < BJ; ++j) {
            const uint8_t* p = stage + tb[j] + blk[st];
#pragma unroll
            for (int x = 0; x < 3; ++x) rb[j][x] = *(const uint2*)(p + 8 * x);
        }
    };
    // acc[j][i] += W_j . X_i^T for one k-step (e2m3 x e2m3, unit scales)
    auto mma = [&](const uint2 (&ra)[BI][3], const uint2 (&rb)[BJ][3]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < BJ; ++j)
#pragma unroll
            for (int i = 0; i < BI; ++i)
                acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fp6_operand(rb[j]), fp6_operand(ra[i]),
                                                                            acc[j][i], 2, 2, 0, 127, 0, 127);
    };
    // each MFMA followed by its share of the phase's fragment reads (two
    // read instructions per fragment: ds_read2_b64 + ds_read_b64)
    auto hints = [&](int reads) __attribute__((always_inline)) {
        constexpr int NM = BI * BJ, NR = 2 * (BI + BJ);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            const int share = ((m + 1) * NR + NM - 1) / NM - (m * NR + NM - 1) / NM;  // 2, 1, ...
            if (reads > 0) {
                if (share == 2)
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                else if (share == 1)
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        }
    };

    // prologue: the epilogue's parameters, then up to three stages in
    // flight; wait for stage 0 (and so for the older parameter copies)
    if constexpr (OUT == GEMM_OUT_BF16)
        issue_epilogue_params<G>(a, tm, tn, wave, lane,
                                 __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)params));
    const int first = KC < G::kStages ? KC : G::kStages;
    for (int st = 0; st < first; ++st) issue(lds0 + st * kStage, kb0 + st);
    if (G::kStages == 3 && first >= 3)
        wait6_and_barrier<G::COPIES, 2>();
    else if (first >= 2)
        wait6_and_barrier<G::COPIES, 1>();
    else
        wait6_and_barrier<G::COPIES, 0>();
    read(smem, 0, xa, xb);

    // One stage.  ISSUE: copy stage kr + 3 into this stage's buffer;
    // IN_FLIGHT: stages that may still be in flight at the barrier; MORE: a
    // stage kr + 1 follows.
    auto step = [&](int kr, auto issue_c, auto in_flight_c, auto more_c) __attribute__((always_inline)) {
        constexpr bool ISSUE = decltype(issue_c)::value != 0;
        constexpr int IN_FLIGHT = decltype(in_flight_c)::value;
        constexpr bool MORE = decltype(more_c)::value != 0;
        const int slot_kr = kr % G::kStages;
        const uint8_t* cur = smem + slot_kr * kStage;
        read(cur, 1, ya, yb);
        mma(xa, xb);
        hints(24);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (MORE) {
            wait6_and_barrier<G::COPIES, IN_FLIGHT>();
            if constexpr (ISSUE) issue(lds0 + slot_kr * kStage, kb0 + kr + G::kStages);
            read(smem + ((kr + 1) % G::kStages) * kStage, 0, xa, xb);
        }
        // no scheduling fence here: the next stage's k-step 0 reads
        // interleave with these MFMAs (issued all at once, they would exceed
        // the 15 LDS reads a wave can have outstanding and stall its MFMAs)
        mma(ya, yb);
        hints(MORE ? 24 : 0);
        __builtin_amdgcn_sched_barrier(0);
    };
    if constexpr (G::kStages == 3) {
        for (int kr = 0; kr < KC - 3; ++kr) step(kr, Const<1>{}, Const<1>{}, Const<1>{});
        if (KC >= 3) step(KC - 3, Const<0>{}, Const<1>{}, Const<1>{});
    } else {
        // two stages: at stage kr's barrier only stage kr + 1 is in flight,
        // and it must have landed; the copy of kr + 2 is issued after it
        for (int kr = 0; kr < KC - 2; ++kr) step(kr, Const<1>{}, Const<0>{}, Const<1>{});
    }
    if (KC >= 2) step(KC - 2, Const<0>{}, Const<0>{}, Const<1>{});
    step(KC - 1, Const<0>{}, Const<0>{}, Const<0>{});

    if constexpr (SPLIT)
        split_k_finish<G, OUT>(a, tile, split, tm, tn, wm, wn, tid, wave, lane, lds0, smem, params, acc);
    else
        gemm_epilogue<G, OUT>(a, tm, tn, wm, wn, tid, wave, lane, smem, params, acc);
}

// ---------------------------------------------------------------------------
// skinny_kernel: M <= 128 (up to four 32-row units of activation codes)
//
// The product is a stream over the weight image.  One workgroup per
// 16-column strip (half of a 32-row weight unit: 1 KB per 128-K unit) and
// 32-row group of activations, its four waves splitting K; each strip is
// computed with the 16x16x64 INT8 MFMA as W . X^T for MH 16-row blocks of
// the group.  Every lane loads one 16-byte chunk (32 codes) of its weight
// row and of its activation row(s) per unit straight into registers -- no
// reuse inside the workgroup, so no LDS staging -- with kSkinnyBatch units of
// loads in flight per wave (at K <= 3072 the whole strip, so the full weight
// image is requested as soon as the grid is resident).  With 16-column
// strips a 12288-column weight is 768 equal workgroups, three per CU.  With
// more than one row group the workgroups of a strip are numbered so that
// they run on the same XCD (workgroups go to the XCDs in turn by number) and
// read the strip from that XCD's L2 after the first.  The activation codes are
// re-read from L2 by every strip.  The chunk of lane quad q feeds k-slots q
// of two MFMAs (its first and second 16 codes); both operands use the same
// assignment, so the sum over k is the dot product.  The four partial tiles
// are summed through LDS and the epilogue writes the valid rows.
// ---------------------------------------------------------------------------

constexpr int kSkinnyWaves = 4;
constexpr int kSkinnyBatch = 6;  // 128-K units per load batch

// 16-byte load of the weight stream.  A plain load: with the non-temporal
// hint the 768-workgroup stream of a 12288 x 3072 weight ran 6% slower
// (5.4 against 5.1 us by kernel trace at M = 16).
__device__ inline uint4 load_stream16(const uint8_t* p) { return *(const uint4*)p; }

// The epilogue's column scales and biases of columns n0 .. n0 + 3 (clamped to
// N - 1, so every lane issues the same loads), requested at the start of a
// kernel so that they are not a chain of dependent round trips at its end.
// No branch around the loads: the wait for a load issued inside a branch
// would also wait for every load issued before it.
__device__ inline void load_column_params(const GemmArgs& a, int64_t n0, float (&swv)[4], float (&bv)[4])
{
    const uint16_t* bsrc = a.bias ? a.bias : (const uint16_t*)a.sw;  // a valid address either way
    const uint32_t bmask = a.bias ? 0xFFFFu : 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t n = min(n0 + j, a.N - 1);
        swv[j] = a.sw[n];
        bv[j] = __uint_as_float(((uint32_t)bsrc[n] & bmask) << 16);
    }
}

// Workgroup number -> (16-column strip, 32-row group) with the groups of a
// strip on one XCD: b = 8 l + x runs on XCD x; l = groups * j + rg.  The
// strips are padded to a multiple of 8; the padding workgroups do nothing.
CONVROT_HD inline int skinny_strips_padded(int64_t N) { return (int)(((N + 15) / 16 + 7) / 8 * 8); }

template <int OUT, int MH>
__global__ __launch_bounds__(kSkinnyWaves * 64) void skinny_kernel(GemmArgs a)
{
    constexpr int BATCH = kSkinnyBatch;
    __shared__ __attribute__((aligned(16))) int32_t red[kSkinnyWaves - 1][MH][4][64];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, q = lane >> 4;
    const int groups = (int)((a.M + 31) / 32);
    const int l = (int)(blockIdx.x >> 3);
    const int rg = l % groups;                                    // rows 32 rg .. 32 rg + 31
    const int strip = (l / groups) * 8 + (int)(blockIdx.x & 7);  // columns 16 strip .. 16 strip + 15
    if ((int64_t)strip * 16 >= a.N) return;  // padding workgroup (uniform exit)
    const int nt = strip >> 1, half = strip & 1;  // weight unit row tile and its half
    const int KB = a.KB;
    const int per = (KB + kSkinnyWaves - 1) / kSkinnyWaves;
    const int kb0 = wave * per, kb1 = min(KB, kb0 + per);
    const int wrow = 16 * half + r16;
    const uint8_t* wbase = a.wgt + (size_t)nt * KB * kUnitBytes + wrow * 64 + ((q ^ row_swizzle(wrow)) * 16);
    const uint8_t* abase[MH];
    bool act_row[MH];
#pragma unroll
    for (int mh = 0; mh < MH; ++mh) {
        const int rr = 16 * mh + r16;  // row of the group's activation unit row tile
        abase[mh] = a.act + (size_t)rg * KB * kUnitBytes + rr * 64 + ((q ^ row_swizzle(rr)) * 16);
        act_row[mh] = 32 * rg + rr < a.M;  // rows past M are zero in the image: not loaded
    }
    // lane's output columns (n0 .. n0 + 3) and rows (32 rg + 16 mh + r16) in the epilogue
    const int64_t n0 = (int64_t)strip * 16 + 4 * q;
    float swv[4], bv[4], sxv[MH];
    if constexpr (OUT == GEMM_OUT_BF16) {
        load_column_params(a, n0, swv, bv);
#pragma unroll
        for (int mh = 0; mh < MH; ++mh) sxv[mh] = a.sx[min((int64_t)(32 * rg + 16 * mh + r16), a.M - 1)];
        __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the weight stream
    }

    v4i acc[MH];
#pragma unroll
    for (int mh = 0; mh < MH; ++mh) acc[mh] = v4i{0, 0, 0, 0};

    for (int kb = kb0; kb < kb1; kb += BATCH) {
        uint4 wq[BATCH], aq[BATCH][MH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const bool in = kb + u < kb1;
            const uint8_t* wp = wbase + (size_t)(kb + u) * kUnitBytes;
            wq[u] = in ? load_stream16(wp) : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int mh = 0; mh < MH; ++mh)
                aq[u][mh] = (in && act_row[mh]) ? *(const uint4*)(abase[mh] + (size_t)(kb + u) * kUnitBytes)
                                                : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            if (kb + u >= kb1) break;
            const v4i w0 = widen_lo_hi(wq[u].x, wq[u].y), w1 = widen_lo_hi(wq[u].z, wq[u].w);
#pragma unroll
            for (int mh = 0; mh < MH; ++mh) {
                acc[mh] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w0, widen_lo_hi(aq[u][mh].x, aq[u][mh].y), acc[mh],
                                                                0, 0, 0);
                acc[mh] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w1, widen_lo_hi(aq[u][mh].z, aq[u][mh].w), acc[mh],
                                                                0, 0, 0);
            }
        }
    }

    // sum the partial tiles of the waves (exact integer sums)
    if (wave > 0) {
#pragma unroll
        for (int mh = 0; mh < MH; ++mh)
#pragma unroll
            for (int j = 0; j < 4; ++j) red[wave - 1][mh][j][lane] = acc[mh][j];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < kSkinnyWaves - 1; ++w)
#pragma unroll
        for (int mh = 0; mh < MH; ++mh)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[mh][j] += red[w][mh][j][lane];

    // lane holds, per block mh, output row m = 32 rg + 16 mh + r16 and the
    // four consecutive columns n = n0 + (0..3)
    if (n0 >= a.N) return;
    const bool vec_ok = (a.N % 4) == 0;
#pragma unroll
    for (int mh = 0; mh < MH; ++mh) {
        const int64_t m = 32 * rg + 16 * mh + r16;
        if (m >= a.M) continue;
        int32_t v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = acc[mh][j] >> 8;  // both operands entered x 16
        if constexpr (OUT == GEMM_OUT_I32) {
            int32_t* dst = (int32_t*)a.out + m * a.N + n0;
            if (vec_ok) {
                *(int4*)dst = make_int4(v[0], v[1], v[2], v[3]);
            } else {
                for (int j = 0; j < 4 && n0 + j < a.N; ++j) dst[j] = v[j];
            }
        } else {
            float y[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) y[j] = __builtin_fmaf((float)v[j] * sxv[mh], swv[j], bv[j]);
            const uint32_t p01 = pack_bf16x2(y[0], y[1]), p23 = pack_bf16x2(y[2], y[3]);
            uint16_t* dst = (uint16_t*)a.out + m * a.N + n0;
            if (vec_ok) {
                *(uint2*)dst = make_uint2(p01, p23);
            } else {
                const uint16_t yb[4] = {(uint16_t)p01, (uint16_t)(p01 >> 16), (uint16_t)p23, (uint16_t)(p23 >> 16)};
                for (int j = 0; j < 4 && n0 + j < a.N; ++j) dst[j] = yb[j];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// w4a16_kernel: weight-only INT4 product for M <= 32 (MH 16-row halves).
//
// Same work split as skinny_kernel -- one workgroup per 16-column strip, its
// four waves splitting K, weight chunks streamed into registers -- but the
// activations are the bf16 rotated rows (no activation codes) and the
// product runs on v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  Lane quad
// q holds 16-byte chunk q of its weight row in a 128-K unit: four words, word
// j being the eight consecutive codes from k = 32 (2 (q / 2) + j / 2) +
// 16 (q % 2) + 8 (j % 2) (the image layout), low nibbles first.  Word j of
// every quad feeds MFMA j, and the activation operand of lane (r, q) is the
// eight bf16 values of row r at the same k: both operands agree on k, so the
// sum over the four MFMAs is the dot product over the unit.  Codes enter as
// the bf16 values 16 q, exactly (each nibble moved to the top of a byte, the
// signed byte converted, pairs packed), so every product and partial sum is
// exactly 16 times that of the codes themselves (binary32 rounding commutes
// with a power of two).  The four partial tiles are summed through LDS in
// wave order and the epilogue is fmaf(acc, sw[n] / 16, bias[n]) rounded to
// bf16, which is fmaf(sum over codes, sw[n], bias[n]).
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// eight INT4 codes q (low nibbles k..k+3, high nibbles k+4..k+7) -> the bf16
// values 16 q in k order.  A nibble at the top of a byte is the signed byte
// 16 q, and the compiler converts a sign-extended byte in one instruction
// (sub-dword operand select): 15 instructions per word instead of 20 for
// extracting each code.
constexpr float kW16CodeScale = 0.0625f;  // 1 / 16: undoes the factor of the operand
__device__ inline bf16x8_t dequant8_bf16(uint32_t w)
{
    const uint32_t lo = (w << 4) & 0xF0F0F0F0u, hi = w & 0xF0F0F0F0u;
    float f[8];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        f[b] = (float)(int8_t)(lo >> (8 * b));
        f[4 + b] = (float)(int8_t)(hi >> (8 * b));
    }
    const uint4 p = make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                               pack_bf16x2(f[6], f[7]));
    return __builtin_bit_cast(bf16x8_t, p);
}

template <int MH, int BATCH>
__global__ __launch_bounds__(kSkinnyWaves * 64) void w4a16_kernel(GemmArgs a, const uint16_t* xr)
{
    __shared__ __attribute__((aligned(16))) float red[kSkinnyWaves - 1][MH][4][64];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, q = lane >> 4;
    const int strip = blockIdx.x;                   // output columns 16 strip .. 16 strip + 15
    const int nt = strip >> 1, half = strip & 1;
    const int KB = a.KB;
    const int per = (KB + kSkinnyWaves - 1) / kSkinnyWaves;
    const int kb0 = wave * per, kb1 = min(KB, kb0 + per);
    const int wrow = 16 * half + r16;
    const uint8_t* wbase = a.wgt + (size_t)nt * KB * kUnitBytes + wrow * 64 + ((q ^ row_swizzle(wrow)) * 16);
    int kst[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) kst[j] = 32 * (2 * (q >> 1) + (j >> 1)) + 16 * (q & 1) + 8 * (j & 1);
    // activation words in the order of w16_word_offset: for 16-row block mh,
    // unit kb and step j, the wave reads 1 KB at ((mh KB + kb) 4 + j) KB + 16 lane
    const uint8_t* xbase[MH];
    bool xok[MH];
#pragma unroll
    for (int mh = 0; mh < MH; ++mh) {
        xok[mh] = 16 * mh + r16 < a.M;
        xbase[mh] = (const uint8_t*)xr + (size_t)mh * KB * 4096 + lane * 16;
    }
    const int64_t n0 = (int64_t)strip * 16 + 4 * q;  // lane's output columns n0 .. n0 + 3
    float swv[4], bv[4];
    load_column_params(a, n0, swv, bv);
    __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the weight stream

    f32x4_t acc[MH];
#pragma unroll
    for (int mh = 0; mh < MH; ++mh) acc[mh] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int kb = kb0; kb < kb1; kb += BATCH) {
        uint4 wq[BATCH];
        uint4 xa[BATCH][4][MH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const bool in = kb + u < kb1;
            wq[u] = in ? load_stream16(wbase + (size_t)(kb + u) * kUnitBytes) : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int mh = 0; mh < MH; ++mh) {
                    const int64_t k = (int64_t)(kb + u) * kTileK + kst[j];
                    xa[u][j][mh] = (in && xok[mh] && k < a.K)
                                       ? *(const uint4*)(xbase[mh] + ((size_t)(kb + u) * 4 + j) * 1024)
                                       : make_uint4(0, 0, 0, 0);
                }
        }
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            if (kb + u >= kb1) break;
            const uint32_t ww[4] = {wq[u].x, wq[u].y, wq[u].z, wq[u].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bf16x8_t wf = dequant8_bf16(ww[j]);
#pragma unroll
                for (int mh = 0; mh < MH; ++mh)
                    acc[mh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, __builtin_bit_cast(bf16x8_t, xa[u][j][mh]),
                                                                      acc[mh], 0, 0, 0);
            }
        }
    }

    // sum the partial tiles of the waves, in wave order
    if (wave > 0) {
#pragma unroll
        for (int mh = 0; mh < MH; ++mh)
#pragma unroll
            for (int j = 0; j < 4; ++j) red[wave - 1][mh][j][lane] = acc[mh][j];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < kSkinnyWaves - 1; ++w)
#pragma unroll
        for (int mh = 0; mh < MH; ++mh)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[mh][j] += red[w][mh][j][lane];

    // lane holds, per half mh, output row m = 16 mh + r16 and the four
    // consecutive columns n = n0 + (0..3)
    if (n0 >= a.N) return;
#pragma unroll
    for (int mh = 0; mh < MH; ++mh) {
        const int64_t m = 16 * mh + r16;
        if (m >= a.M) continue;
        float y[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = __builtin_fmaf(acc[mh][j], swv[j] * kW16CodeScale, bv[j]);
        const uint32_t p01 = pack_bf16x2(y[0], y[1]), p23 = pack_bf16x2(y[2], y[3]);
        uint16_t* dst = (uint16_t*)a.out + m * a.N + n0;
        if ((a.N % 4) == 0) {
            *(uint2*)dst = make_uint2(p01, p23);
        } else {
            const uint16_t yb[4] = {(uint16_t)p01, (uint16_t)(p01 >> 16), (uint16_t)p23, (uint16_t)(p23 >> 16)};
            for (int j = 0; j < 4 && n0 + j < a.N; ++j) dst[j] = yb[j];
        }
    }
}

// ---------------------------------------------------------------------------
// small_m_kernel: the whole linear in one launch for M <= kSmallRows, when a
// row's prep team is whole waves (64 <= K / P <= 256).
//
// A workgroup owns SW 16-column strips, four waves per strip splitting K as
// in skinny_kernel.  It first requests its whole weight range (every wave's
// loads in flight), then -- while the weights stream in -- computes the
// activation codes of all M rows itself, with the prep kernel's rotation and
// quantization, into its own shared memory: a team of K / (64 P) waves per
// row, several rows at once.  Every workgroup repeats this small prep (M rows
// of at most 4096 values: a few microseconds of vector work over the whole
// GPU, hidden under the memory-bound weight stream), which needs no exchange
// between workgroups at all.  Then the MFMAs read the codes from shared
// memory, and each strip's four partial tiles are reduced and stored as in
// skinny_kernel.  Workgroup 0 also writes the codes and scales to the
// workspace, as the two-kernel path leaves them there.
// ---------------------------------------------------------------------------
constexpr int kSmallUnits = 8;     // 128-K units per wave: K <= 4096 over four waves

template <int G, int SW, bool REG>
__global__ __launch_bounds__(SW * kSkinnyWaves * 64) void small_m_kernel(GemmArgs a, PrepArgs p)
{
    using PS = PrepShape<G>;
    constexpr int P = PS::P;
    constexpr int NWAVES = SW * kSkinnyWaves;
    __shared__ __attribute__((aligned(16))) uint8_t plds[NWAVES * PS::kWaveLdsBytes];
    __shared__ uint32_t pred[2][16];
    __shared__ __attribute__((aligned(16))) uint8_t act[kSmallUnits * kSkinnyWaves * kSmallRows * 64];
    __shared__ float sxl[kSmallRows];
    __shared__ __attribute__((aligned(16))) int32_t red[SW][kSkinnyWaves - 1][4][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int sl = wave / kSkinnyWaves, kq = wave % kSkinnyWaves;  // strip within the workgroup, K quarter
    const int r16 = lane & 15, q = lane >> 4;
    const int strip = blockIdx.x * SW + sl;
    const int nstrips = (int)((a.N + 15) / 16);
    const int strip_c = min(strip, nstrips - 1);  // past the end: re-read the last strip, never stored
    const int nt = strip_c >> 1, half = strip_c & 1;
    const int KB = a.KB;
    const int per = (KB + kSkinnyWaves - 1) / kSkinnyWaves;  // <= kSmallUnits
    const int kb0 = kq * per;
    const int kn = max(0, min(KB, kb0 + per) - kb0);          // units of this wave
    const int wrow = 16 * half + r16;
    const uint8_t* wbase = a.wgt + (size_t)nt * KB * kUnitBytes + wrow * 64 + ((q ^ row_swizzle(wrow)) * 16);

    // prep teams: K / (64 P) waves per activation row, `teams` rows at a time
    const int team_nw = (int)(p.K_pad / P + 63) / 64;  // waves per row
    const int teams = NWAVES / team_nw;
    const int team = wave / team_nw;
    const bool live = team < teams;  // waves past the last whole team only take part in the barriers
    const int t = tid - team * team_nw * 64;           // lane within the team
    const int64_t k0 = (int64_t)t * P;

    // 1. the activation values of the first pass, then the wave's whole weight
    //    range, all in flight (weight units past the wave's range re-read its
    //    last unit and are not used, so every path issues the same number of
    //    loads -- and the wait for the activation values, issued first, does
    //    not wait for the weights)
    uint4 xw[P / 8];
    load_run<P>(p.X, live ? team : 0, p.ld, k0, live && team < p.rows, xw);
    // the epilogue's column scales and biases (clamped columns: every lane
    // issues the same loads; only the first wave of each strip uses them)
    const int64_t n0 = (int64_t)strip * 16 + 4 * q;
    float swv[4], bv[4];
    load_column_params(a, n0, swv, bv);
    __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the weight loads
    uint4 wq[kSmallUnits];
#pragma unroll
    for (int u = 0; u < kSmallUnits; ++u) {
        const int kb = min(kb0 + min(u, max(kn - 1, 0)), KB - 1);
        wq[u] = load_stream16(wbase + (size_t)kb * kUnitBytes);
    }

    // 2. activation codes of the M rows into shared memory (the first pass is
    //    outside the loop: a load inside the loop body would make the wait for
    //    the first pass's values also wait for the weights).  Only rows < M
    //    are computed -- the products never read the others -- and a team
    //    without a row still takes the team-absmax barrier of prep_row.
    {
        double* ld = (double*)(plds + wave * PS::kWaveLdsBytes);
        PrepArgs pl = p;
        pl.out = act;     // codes and scales go to this workgroup's shared memory
        pl.scales = sxl;
        const int passes = (int)((a.M + teams - 1) / teams);  // rows 0 .. M - 1
        if (live && team < a.M)  // uniform over the team's waves
            prep_row<G, OUT_LDS, kSmallRows, REG>(pl, xw, team, t, k0, lane, wave, ld, pred, 0, team * team_nw,
                                                   team_nw);
        else if (p.team > 64)
            __syncthreads();
        for (int pass = 1; pass < passes; ++pass) {
            const int64_t row = (int64_t)pass * teams + (live ? team : 0);
            const bool active = live && row < a.M;
            load_run<P>(p.X, row, p.ld, k0, active, xw);
            if (active)
                prep_row<G, OUT_LDS, kSmallRows, REG>(pl, xw, row, t, k0, lane, wave, ld, pred, pass & 1, team * team_nw,
                                                  team_nw);
            else if (p.team > 64)
                __syncthreads();
        }
    }
    __syncthreads();
    if (blockIdx.x == 0) {
        // the workspace also receives the codes and scales (rows 0 .. M-1 of the
        // image's first row tile; same in-row layout)
        const int words = KB * (int)a.M * 4;  // 16-byte words
        for (int i = tid; i < words; i += NWAVES * 64) {
            const int kb = i / ((int)a.M * 4), r = (i / 4) % (int)a.M, c = i % 4;
            *(uint4*)(p.out + (size_t)kb * kUnitBytes + r * 64 + c * 16) =
                *(const uint4*)(act + (kb * kSmallRows + r) * 64 + c * 16);
        }
        if (tid < a.M) p.scales[tid] = sxl[tid];
    }

    // 3. products: weights from registers, activation codes from shared memory
    const bool act_row = r16 < a.M;
    v4i acc = v4i{0, 0, 0, 0}, acc1 = v4i{0, 0, 0, 0};  // two chains of dependent MFMAs
#pragma unroll
    for (int u = 0; u < kSmallUnits; ++u) {
        if (u >= kn) break;
        uint4 x = make_uint4(0, 0, 0, 0);
        if (act_row) x = *(const uint4*)(act + ((kb0 + u) * kSmallRows + r16) * 64 + ((q ^ row_swizzle(r16)) * 16));
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(widen_lo_hi(wq[u].x, wq[u].y), widen_lo_hi(x.x, x.y), acc, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(widen_lo_hi(wq[u].z, wq[u].w), widen_lo_hi(x.z, x.w), acc1, 0, 0, 0);
    }
    acc += acc1;

    // 4. reduce each strip's partial tiles, store
    if (kq > 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) red[sl][kq - 1][j][lane] = acc[j];
    }
    __syncthreads();
    if (kq != 0) return;
#pragma unroll
    for (int w = 0; w < kSkinnyWaves - 1; ++w)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] += red[sl][w][j][lane];
    const int64_t m = r16;
    if (n0 >= a.N || m >= a.M) return;
    const float sxm = sxl[m];
    float y[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) y[j] = __builtin_fmaf((float)(acc[j] >> 8) * sxm, swv[j], bv[j]);  // operands x 16
    const uint32_t p01 = pack_bf16x2(y[0], y[1]), p23 = pack_bf16x2(y[2], y[3]);
    uint16_t* dst = (uint16_t*)a.out + m * a.N + n0;
    if ((a.N % 4) == 0) {
        *(uint2*)dst = make_uint2(p01, p23);
    } else {
        const uint16_t yb[4] = {(uint16_t)p01, (uint16_t)(p01 >> 16), (uint16_t)p23, (uint16_t)(p23 >> 16)};
        for (int j = 0; j < 4 && n0 + j < a.N; ++j) dst[j] = yb[j];
    }
}

// ---------------------------------------------------------------------------
// small_w4a16_kernel: the W4A16 linear in one launch, for the shapes of the
// single-kernel W4A4 linear (M <= kSmallRows, a row's prep team whole waves).
//
// As in small_m_kernel, a workgroup first requests its whole weight range and,
// while the weights stream in, rotates the M activation rows itself -- here
// rounded to bf16, as the prep kernel's bf16 mode writes them -- into its own
// shared memory.  The products then run exactly as in w4a16_kernel (the same
// split of K over the four waves, the same MFMA order, the partial tiles
// summed in wave order), with the activation operand from shared memory, so
// the result equals the two-launch path's bit for bit.  Workgroup 0 also
// writes the bf16 rows to the workspace.
// ---------------------------------------------------------------------------
template <int G, int SW, bool REG>
__global__ __launch_bounds__(SW * kSkinnyWaves * 64) void small_w4a16_kernel(GemmArgs a, PrepArgs p)
{
    using PS = PrepShape<G>;
    constexpr int P = PS::P;
    constexpr int NWAVES = SW * kSkinnyWaves;
    constexpr int kMaxRowK = kSmallUnits * kSkinnyWaves * kTileK;  // longest row: 4096 values
    __shared__ __attribute__((aligned(16))) uint8_t plds[NWAVES * PS::kWaveLdsBytes];
    __shared__ uint32_t pred[2][16];
    __shared__ __attribute__((aligned(16))) uint16_t xr[kSmallRows * kMaxRowK];  // bf16 rows, K values apart
    __shared__ __attribute__((aligned(16))) float red[SW][kSkinnyWaves - 1][4][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int sl = wave / kSkinnyWaves, kq = wave % kSkinnyWaves;  // strip within the workgroup, K quarter
    const int r16 = lane & 15, q = lane >> 4;
    const int strip = blockIdx.x * SW + sl;
    const int nstrips = (int)((a.N + 15) / 16);
    const int strip_c = min(strip, nstrips - 1);  // past the end: re-read the last strip, never stored
    const int nt = strip_c >> 1, half = strip_c & 1;
    const int KB = a.KB;
    const int per = (KB + kSkinnyWaves - 1) / kSkinnyWaves;  // <= kSmallUnits
    const int kb0 = kq * per;
    const int kn = max(0, min(KB, kb0 + per) - kb0);          // units of this wave
    const int wrow = 16 * half + r16;
    const uint8_t* wbase = a.wgt + (size_t)nt * KB * kUnitBytes + wrow * 64 + ((q ^ row_swizzle(wrow)) * 16);

    const int team_nw = (int)(p.K_pad / P + 63) / 64;  // waves per row
    const int teams = NWAVES / team_nw;
    const int team = wave / team_nw;
    const bool live = team < teams;
    const int t = tid - team * team_nw * 64;
    const int64_t k0 = (int64_t)t * P;

    // 1. the first pass's activation values, the epilogue's scales and
    //    biases, then the whole weight range: all in flight
    uint4 xw[P / 8];
    load_run<P>(p.X, live ? team : 0, p.ld, k0, live && team < p.rows, xw);
    const int64_t n0 = (int64_t)strip * 16 + 4 * q;
    float swv[4], bv[4];
    load_column_params(a, n0, swv, bv);
    __builtin_amdgcn_sched_barrier(0);
    uint4 wq[kSmallUnits];
#pragma unroll
    for (int u = 0; u < kSmallUnits; ++u) {
        const int kb = min(kb0 + min(u, max(kn - 1, 0)), KB - 1);
        wq[u] = load_stream16(wbase + (size_t)kb * kUnitBytes);
    }

    // 2. the bf16 rotated rows 0 .. M-1 into shared memory (the bf16 mode has
    //    no team barrier: teams without a row skip it)
    {
        double* ld = (double*)(plds + wave * PS::kWaveLdsBytes);
        PrepArgs pl = p;
        pl.out = (uint8_t*)xr;
        const int passes = (int)((a.M + teams - 1) / teams);
        if (live && team < a.M)
            prep_row<G, OUT_ROTATED_BF16, kSmallRows, REG>(pl, xw, team, t, k0, lane, wave, ld, pred, 0,
                                                           team * team_nw, team_nw);
        for (int pass = 1; pass < passes; ++pass) {
            const int64_t row = (int64_t)pass * teams + (live ? team : 0);
            const bool active = live && row < a.M;
            load_run<P>(p.X, row, p.ld, k0, active, xw);
            if (active)
                prep_row<G, OUT_ROTATED_BF16, kSmallRows, REG>(pl, xw, row, t, k0, lane, wave, ld, pred, pass & 1,
                                                               team * team_nw, team_nw);
        }
    }
    __syncthreads();
    if (blockIdx.x == 0) {  // the rows into the workspace, in the two-launch path's order
        const int row_words = (int)(a.K / 8);  // 16-byte words of a row
        for (int i = tid; i < (int)a.M * row_words; i += NWAVES * 64) {
            const int m = i / row_words, k = (i % row_words) * 8;
            *(uint4*)(p.out + w16_word_offset(m, k, a.K)) = ((const uint4*)xr)[i];
        }
    }

    // 3. products, as in w4a16_kernel (MH = 1)
    int kst[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) kst[j] = 32 * (2 * (q >> 1) + (j >> 1)) + 16 * (q & 1) + 8 * (j & 1);
    const bool act_row = r16 < a.M;
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kSmallUnits; ++u) {
        if (u >= kn) break;
        const uint32_t ww[4] = {wq[u].x, wq[u].y, wq[u].z, wq[u].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t k = (int64_t)(kb0 + u) * kTileK + kst[j];
            const uint4 x = (act_row && k < a.K) ? *(const uint4*)(xr + r16 * a.K + k) : make_uint4(0, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dequant8_bf16(ww[j]), __builtin_bit_cast(bf16x8_t, x), acc,
                                                          0, 0, 0);
        }
    }

    // 4. the strip's partial tiles summed in wave order, epilogue
    if (kq > 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) red[sl][kq - 1][j][lane] = acc[j];
    }
    __syncthreads();
    if (kq != 0) return;
#pragma unroll
    for (int w = 0; w < kSkinnyWaves - 1; ++w)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] += red[sl][w][j][lane];
    const int64_t m = r16;
    if (n0 >= a.N || m >= a.M) return;
    float y[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) y[j] = __builtin_fmaf(acc[j], swv[j] * kW16CodeScale, bv[j]);
    const uint32_t p01 = pack_bf16x2(y[0], y[1]), p23 = pack_bf16x2(y[2], y[3]);
    uint16_t* dst = (uint16_t*)a.out + m * a.N + n0;
    if ((a.N % 4) == 0) {
        *(uint2*)dst = make_uint2(p01, p23);
    } else {
        const uint16_t yb[4] = {(uint16_t)p01, (uint16_t)(p01 >> 16), (uint16_t)p23, (uint16_t)(p23 >> 16)};
        for (int j = 0; j < 4 && n0 + j < a.N; ++j) dst[j] = yb[j];
    }
}

// ---------------------------------------------------------------------------
// layout kernels
// ---------------------------------------------------------------------------

// The FP6 fields of codes k .. k+7 (code e at bits 6 e) into the FP6 image:
// three 16-bit pieces from logical byte 24 (k % 128 / 32) + 6 (k % 32 / 8).
__device__ inline void store_fp6_8(uint8_t* image6, int64_t row, int64_t k, int64_t K_pad, const int (&q)[8])
{
    uint64_t v = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) v |= (uint64_t)fp6_e2m3(q[e]) << (6 * e);
    const int kl = (int)(k % kTileK);
    const int b0 = 24 * (kl / 32) + 6 * ((kl % 32) / 8);
#pragma unroll
    for (int d = 0; d < 3; ++d)
        *(uint16_t*)(image6 + image6_byte_offset(row, k / kTileK, b0 + 2 * d, K_pad)) = (uint16_t)(v >> (16 * d));
}

// int8 codes [M][K] -> operand images (zero padding); one thread per 8 codes.
__global__ void act_relayout_kernel(const int8_t* codes, int64_t M, int64_t K, int64_t M_pad, int64_t K_pad,
                                    uint8_t* image, uint8_t* image6, uint32_t* zero, int zero_count)
{
    const int64_t words_per_row = K_pad / 8;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t < zero_count) zero[t] = 0;  // split-K counters of the GEMM that consumes this workspace
    if (t >= M_pad * words_per_row) return;
    const int64_t m = t / words_per_row, k = (t % words_per_row) * 8;
    uint32_t out = 0;
    int q[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (m < M && k < K) {
        const uint2 in = *(const uint2*)(codes + m * K + k);  // codes k..k+7, one per byte
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint32_t c_lo = (in.x >> (8 * b)) & 0xFu;  // code k + b
            const uint32_t c_hi = (in.y >> (8 * b)) & 0xFu;  // code k + 4 + b
            out |= (c_lo | (c_hi << 4)) << (8 * b);
            q[b] = (int)(int8_t)(in.x >> (8 * b));
            q[4 + b] = (int)(int8_t)(in.y >> (8 * b));
        }
    }
    *(uint32_t*)(image + image_word_offset(m, k, K_pad)) = out;
    if (image6) store_fp6_8(image6, m, k, K_pad, q);
}

// N x packed-K [N][K/2] -> operand images (zero padding); one thread per 8 codes.
__global__ void repack_nk_kernel(const uint8_t* nk, int64_t N, int64_t K, int64_t N_pad, int64_t K_pad,
                                 uint8_t* image, uint8_t* image6)
{
    const int64_t words_per_col = K_pad / 8;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= N_pad * words_per_col) return;
    const int64_t n = t / words_per_col, k = (t % words_per_col) * 8;
    uint32_t out = 0;
    int q[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (n < N && k < K) {
        const uint32_t in = *(const uint32_t*)(nk + n * (K / 2) + k / 2);  // codes k..k+7, two per byte
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint32_t c_lo = (in >> (4 * b)) & 0xFu;        // code k + b
            const uint32_t c_hi = (in >> (4 * (b + 4))) & 0xFu;  // code k + 4 + b
            out |= (c_lo | (c_hi << 4)) << (8 * b);
            q[b] = ((int)(c_lo << 28)) >> 28;
            q[4 + b] = ((int)(c_hi << 28)) >> 28;
        }
    }
    *(uint32_t*)(image + image_word_offset(n, k, K_pad)) = out;
    if (image6) store_fp6_8(image6, n, k, K_pad, q);
}

// ---------------------------------------------------------------------------
// host-side launchers
// ---------------------------------------------------------------------------

// Compute units of the current device (cached per device).
static int device_cus()
{
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

template <int G, int MODE, bool REG>
static void launch_prep_g(PrepArgs a, hipStream_t s)
{
    constexpr int P = PrepShape<G>::P;
    const int lanes = (int)(a.K_pad / P);  // lanes per row
    int team = 1;
    int block;
    int64_t row_slots;  // rows one workgroup holds at a time
    if (lanes <= 64) {
        while (team < lanes) team <<= 1;
        block = 256;
        row_slots = 256 / team;
    } else {
        team = (lanes + 63) / 64 * 64;
        block = team;
        row_slots = 1;
    }
    a.team = team;
    const size_t lds = (size_t)(block / 64) * PrepShape<G>::kWaveLdsBytes;
    static bool attr_set = false;  // benign race: every caller sets the same value
    if (!attr_set) {
        (void)hipFuncSetAttribute((const void*)&prep_kernel<G, MODE, REG>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  16 * PrepShape<G>::kWaveLdsBytes);
        attr_set = true;
    }
    // One resident grid's worth of workgroups at most; each walks its rows
    // with a stride of the grid.
    static std::atomic<int> per_cu_cache[17];  // by waves per workgroup
    const int waves = block / 64;
    int per_cu = per_cu_cache[waves].load(std::memory_order_relaxed);
    if (per_cu == 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)&prep_kernel<G, MODE, REG>, block, lds) !=
                hipSuccess ||
            per_cu <= 0)
            per_cu = 1;
        per_cu_cache[waves].store(per_cu, std::memory_order_relaxed);
    }
    const int64_t need = (a.rows_pad + row_slots - 1) / row_slots;
    const int64_t resident = (int64_t)device_cus() * per_cu;
    const unsigned grid = (unsigned)(need < resident ? need : resident);
    hipLaunchKernelGGL((prep_kernel<G, MODE, REG>), dim3(grid), dim3(block), lds, s, a);
}

// Workgroups of one kernel instance resident per compute unit (cached per
// instance and block size).
template <typename KernelPtr>
static int resident_per_cu(KernelPtr kernel, int block, size_t lds, std::atomic<int> (&cache)[17])
{
    const int waves = block / 64;
    int per_cu = cache[waves].load(std::memory_order_relaxed);
    if (per_cu == 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)kernel, block, lds) != hipSuccess ||
            per_cu <= 0)
            per_cu = 1;
        cache[waves].store(per_cu, std::memory_order_relaxed);
    }
    return per_cu;
}

template <int G, bool REG, bool OUT4, bool OUT6, bool ONE_ROW>
static int prep_team_resident(int team, size_t lds)
{
    static bool attr_set = false;  // benign race: every caller sets the same value
    if (!attr_set) {
        (void)hipFuncSetAttribute((const void*)&prep_team_kernel<G, REG, OUT4, OUT6, ONE_ROW>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 16 * PrepShape<G>::kWaveLdsBytes);
        attr_set = true;
    }
    static std::atomic<int> cache[17];
    return device_cus() * resident_per_cu(&prep_team_kernel<G, REG, OUT4, OUT6, ONE_ROW>, team, lds, cache);
}

// When the resident grid of the one-row instance covers every row, each row
// gets a workgroup of its own (no prefetch registers, more waves per SIMD);
// otherwise one resident grid's worth of workgroups walks the rows.
template <int G, bool REG, bool OUT4, bool OUT6>
static void launch_prep_team(const PrepArgs& a, int team, hipStream_t s)
{
    const size_t lds = (size_t)(team / 64) * PrepShape<G>::kWaveLdsBytes;
    if (a.rows_pad <= prep_team_resident<G, REG, OUT4, OUT6, true>(team, lds)) {
        hipLaunchKernelGGL((prep_team_kernel<G, REG, OUT4, OUT6, true>), dim3((unsigned)a.rows_pad), dim3(team), lds,
                           s, a);
        return;
    }
    const int64_t resident = prep_team_resident<G, REG, OUT4, OUT6, false>(team, lds);
    const unsigned grid = (unsigned)(a.rows_pad < resident ? a.rows_pad : resident);
    hipLaunchKernelGGL((prep_team_kernel<G, REG, OUT4, OUT6, false>), dim3(grid), dim3(team), lds, s, a);
}

template <int G, bool REG>
static void launch_prep_team_out(PrepArgs a, hipStream_t s)
{
    constexpr int P = PrepShape<G>::P;
    const int team = (int)((a.K_pad / P + 63) / 64 * 64);
    a.team = team;
    if (a.out && a.out6)
        launch_prep_team<G, REG, true, true>(a, team, s);
    else if (a.out)
        launch_prep_team<G, REG, true, false>(a, team, s);
    else
        launch_prep_team<G, REG, false, true>(a, team, s);
}

template <int MODE>
static void launch_prep_mode(int g, const PrepArgs& a, hipStream_t s)
{
    if constexpr (MODE == OUT_IMAGE) {
        // rows of whole waves: the team kernel (scalar row addressing)
        const bool reg = (g & kRegularHadamard) != 0;
        const int gs = group_size(g);
        if (a.K_pad / (gs == 256 ? 16 : 8) > 64) {
            if (gs == 256)
                reg ? launch_prep_team_out<256, true>(a, s) : launch_prep_team_out<256, false>(a, s);
            else
                reg ? launch_prep_team_out<64, true>(a, s) : launch_prep_team_out<64, false>(a, s);
            return;
        }
    }
    const bool reg = (g & kRegularHadamard) != 0;
    g = group_size(g);
    if (g == 256)
        reg ? launch_prep_g<256, MODE, true>(a, s) : launch_prep_g<256, MODE, false>(a, s);
    else
        reg ? launch_prep_g<64, MODE, true>(a, s) : launch_prep_g<64, MODE, false>(a, s);
}

void launch_prep(int g, int mode, PrepArgs a, hipStream_t s)
{
    switch (mode) {
        case OUT_IMAGE: launch_prep_mode<OUT_IMAGE>(g, a, s); break;
        case OUT_NK: launch_prep_mode<OUT_NK>(g, a, s); break;
        case OUT_ROTATED_BF16: launch_prep_mode<OUT_ROTATED_BF16>(g, a, s); break;
        default: launch_prep_mode<OUT_ROWMAJOR>(g, a, s); break;
    }
}

// one or two 16-row blocks of each 32-row group per workgroup
template <int OUT>
static void launch_skinny(const GemmArgs& a, hipStream_t s)
{
    const int groups = (int)((a.M + 31) / 32);
    const dim3 grid((unsigned)(skinny_strips_padded(a.N) * groups)), block(kSkinnyWaves * 64);
    if (a.M <= 16)
        hipLaunchKernelGGL((skinny_kernel<OUT, 1>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((skinny_kernel<OUT, 2>), grid, block, 0, s, a);
}

template <typename G, int OUT, bool SPLIT>
static void launch_block_tile_kernel(dim3 grid, const GemmArgs& a, hipStream_t s)
{
    if constexpr (gemm_shape_fp6(G::SHAPE))
        hipLaunchKernelGGL((gemm6_kernel<OUT, G, SPLIT>), grid, dim3(G::NW * 64), 0, s, a);
    else
        hipLaunchKernelGGL((gemm_kernel<OUT, G::SHAPE, SPLIT>), grid, dim3(G::NW * 64), 0, s, a);
}

template <typename G>
static void launch_block_tile(int out_mode, bool split, dim3 grid, const GemmArgs& a, hipStream_t s)
{
    if (out_mode == GEMM_OUT_I32)
        split ? launch_block_tile_kernel<G, GEMM_OUT_I32, true>(grid, a, s)
              : launch_block_tile_kernel<G, GEMM_OUT_I32, false>(grid, a, s);
    else
        split ? launch_block_tile_kernel<G, GEMM_OUT_BF16, true>(grid, a, s)
              : launch_block_tile_kernel<G, GEMM_OUT_BF16, false>(grid, a, s);
}

void launch_gemm(int out_mode, GemmArgs a, hipStream_t s)
{
    if (a.M <= kStreamMaxRows) {
        if (out_mode == GEMM_OUT_I32)
            launch_skinny<GEMM_OUT_I32>(a, s);
        else
            launch_skinny<GEMM_OUT_BF16>(a, s);
        return;
    }
    if (a.splits < 1) a.splits = 1;
    const dim3 grid((unsigned)(a.tiles_m * a.tiles_n * a.splits));
    const bool split = a.splits > 1;
    if (a.shape == 2)
        launch_block_tile<Gemm6W8>(out_mode, split, grid, a, s);
    else if (a.shape == 3)
        launch_block_tile<Gemm6Wide>(out_mode, split, grid, a, s);
    else if (a.shape == 0)
        launch_block_tile<GemmGeom<0>>(out_mode, split, grid, a, s);
    else
        launch_block_tile<GemmGeom<1>>(out_mode, split, grid, a, s);
}

template <int G, bool REG>
static void launch_small_m_g(int sw, const GemmArgs& a, const PrepArgs& p, dim3 grid, hipStream_t s)
{
    switch (sw) {
        case 1: hipLaunchKernelGGL((small_m_kernel<G, 1, REG>), grid, dim3(1 * kSkinnyWaves * 64), 0, s, a, p); break;
        case 2: hipLaunchKernelGGL((small_m_kernel<G, 2, REG>), grid, dim3(2 * kSkinnyWaves * 64), 0, s, a, p); break;
        default: hipLaunchKernelGGL((small_m_kernel<G, 3, REG>), grid, dim3(3 * kSkinnyWaves * 64), 0, s, a, p); break;
    }
}

void launch_small_m(int g, GemmArgs a, PrepArgs p, hipStream_t s)
{
    // strips per workgroup: about one workgroup per compute unit, at most 3
    const int64_t strips = (a.N + 15) / 16;
    const int cus = device_cus();
    const int sw = (int)std::min<int64_t>(3, std::max<int64_t>(1, (strips + cus - 1) / cus));
    const bool reg = (g & kRegularHadamard) != 0;
    g = group_size(g);
    p.team = (int)(p.K_pad / (g == 256 ? 16 : 8));  // lanes per row (whole waves: 64 .. 256)
    p.rows_pad = kSmallRows;
    const dim3 grid((unsigned)((strips + sw - 1) / sw));
    if (g == 256)
        reg ? launch_small_m_g<256, true>(sw, a, p, grid, s) : launch_small_m_g<256, false>(sw, a, p, grid, s);
    else
        reg ? launch_small_m_g<64, true>(sw, a, p, grid, s) : launch_small_m_g<64, false>(sw, a, p, grid, s);
}

template <int G, bool REG>
static void launch_small_w4a16_g(int sw, const GemmArgs& a, const PrepArgs& p, dim3 grid, hipStream_t s)
{
    switch (sw) {
        case 1: hipLaunchKernelGGL((small_w4a16_kernel<G, 1, REG>), grid, dim3(1 * kSkinnyWaves * 64), 0, s, a, p); break;
        case 2: hipLaunchKernelGGL((small_w4a16_kernel<G, 2, REG>), grid, dim3(2 * kSkinnyWaves * 64), 0, s, a, p); break;
        default: hipLaunchKernelGGL((small_w4a16_kernel<G, 3, REG>), grid, dim3(3 * kSkinnyWaves * 64), 0, s, a, p); break;
    }
}

void launch_small_w4a16(int g, GemmArgs a, PrepArgs p, hipStream_t s)
{
    const int64_t strips = (a.N + 15) / 16;
    const int cus = device_cus();
    const int sw = (int)std::min<int64_t>(3, std::max<int64_t>(1, (strips + cus - 1) / cus));
    const bool reg = (g & kRegularHadamard) != 0;
    g = group_size(g);
    p.team = (int)(p.K_pad / (g == 256 ? 16 : 8));
    p.rows_pad = kSmallRows;
    const dim3 grid((unsigned)((strips + sw - 1) / sw));
    if (g == 256)
        reg ? launch_small_w4a16_g<256, true>(sw, a, p, grid, s) : launch_small_w4a16_g<256, false>(sw, a, p, grid, s);
    else
        reg ? launch_small_w4a16_g<64, true>(sw, a, p, grid, s) : launch_small_w4a16_g<64, false>(sw, a, p, grid, s);
}

void launch_w4a16(GemmArgs a, const uint16_t* xr, hipStream_t s)
{
    const dim3 grid((unsigned)((a.N + 15) / 16)), block(kSkinnyWaves * 64);
    if (a.M <= 16)
        hipLaunchKernelGGL((w4a16_kernel<1, 6>), grid, block, 0, s, a, xr);
    else
        hipLaunchKernelGGL((w4a16_kernel<2, 3>), grid, block, 0, s, a, xr);
}

void launch_act_relayout(const int8_t* codes, int64_t M, int64_t K, uint8_t* image, uint8_t* image6, uint32_t* zero,
                         int zero_count, hipStream_t s)
{
    const int64_t M_pad = round_up(M, kTileRows), K_pad = round_up(K, kTileK);
    int64_t n = M_pad * (K_pad / 8);
    if (n < zero_count) n = zero_count;
    hipLaunchKernelGGL(act_relayout_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, codes, M, K, M_pad,
                       K_pad, image, image6, zero, zero_count);
}

void launch_repack_nk(const uint8_t* nk, int64_t N, int64_t K, uint8_t* image, uint8_t* image6, hipStream_t s)
{
    const int64_t N_pad = round_up(N, kTileRows), K_pad = round_up(K, kTileK);
    const int64_t n = N_pad * (K_pad / 8);
    hipLaunchKernelGGL(repack_nk_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, nk, N, K, N_pad, K_pad,
                       image, image6);
}

// ---------------------------------------------------------------------------
// Matrix-core rate probe (a measurement hook): each wave runs `iters` rounds
// of four independent MFMA chains on operands held in registers -- no memory
// traffic in the loop -- and stores one value per lane at the end.  Two
// workgroups of four waves per CU: two waves per SIMD, as the block tiles.
// The rate it reaches is the practical denominator beside the published peak
// (the clock under sustained matrix-core load is below the 2.4 GHz of the
// peak figure).
// ---------------------------------------------------------------------------
template <int KIND>
__global__ __launch_bounds__(kProbeThreads) void mfma_rate_kernel(float* out, int iters, int seed)
{
    const int lane = threadIdx.x & 63;
    v8i a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = seed * (lane + i);
        b[i] = seed ^ (lane * 3 + i);
    }
    v16f acc[4];
    v16i iacc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            acc[t][r] = 0.0f;
            iacc[t][r] = 0;
        }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if constexpr (KIND == kProbeFp6) {
                acc[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[t], 2, 2, 0, 127, 0, 127);
            } else {
                const v4i a4 = {a[0], a[1], a[2], a[3]}, b4 = {b[0], b[1], b[2], b[3]};
                iacc[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a4, b4, iacc[t], 0, 0, 0);
            }
        }
    }
    float sum = 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += acc[t][r] + (float)iacc[t][r];
    out[blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

int64_t probe_grid() { return 2 * (int64_t)device_cus(); }

void launch_mfma_probe(int kind, int iters, float* out, hipStream_t s)
{
    const dim3 grid((unsigned)probe_grid()), block(kProbeThreads);
    if (kind == kProbeFp6)
        hipLaunchKernelGGL((mfma_rate_kernel<kProbeFp6>), grid, block, 0, s, out, iters, 3);
    else
        hipLaunchKernelGGL((mfma_rate_kernel<kProbeInt8>), grid, block, 0, s, out, iters, 3);
}

}  // namespace convrot
