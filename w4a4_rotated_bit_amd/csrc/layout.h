// layout.h -- byte layout of the ConvRot W4A4 operands in device memory.
//
// Both GEMM operands -- the activation codes (rows m) and the weight codes
// (rows n, i.e. output channels) -- are stored as the same "operand image" of
// signed INT4 codes, two per byte.  The image is laid out so that the GEMM
// moves it with straight 16-byte copies (global memory -> LDS) and reads MFMA
// fragments out of LDS without bank conflicts.
//
//   unit (rt, kb) = rows [32 rt, 32 rt + 32) x k [128 kb, 128 kb + 128),
//   2048 bytes at ((rt * KB) + kb) * 2048, KB = K_pad / 128; the units of one
//   32-row strip are consecutive along K, so a strip streams linearly.
//   Row r of a unit owns bytes [64 r, 64 r + 64): four 16-byte chunks; logical
//   chunk ch = 2 p + h (p = pair of 32-wide k-steps, h = half of a k-step) is
//   stored at chunk position ch ^ row_swizzle(r) and holds
//     bytes 0..7 : k-step 2p,   codes k = 32(2p)   + 16h + t, t = 0..15
//     bytes 8..15: k-step 2p+1, codes k = 32(2p+1) + 16h + t, t = 0..15
//   Within each 8-byte group, dword d (0..1) byte b (0..3) holds code
//   t = 8d + b in its low nibble and code t = 8d + 4 + b in its high nibble,
//   so that (dword << 4) & 0xF0F0F0F0 and dword & 0xF0F0F0F0 are the codes
//   t = 8d + (0..3) and 8d + (4..7) as INT8 values times 16, in natural order:
//   exactly the 16 bytes one lane feeds to a 32x32x32 INT8 MFMA for k-step
//   2p + (0 or 1), half h.
//
// Padding: rows up to a multiple of 32 and K up to a multiple of 128 are
// stored as code 0.
//
// Swizzle: a fragment read (ds_read_b128) has the 32 lanes of one half wave
// read the same logical chunk of 32 consecutive rows.  The swizzle gives every
// 8 consecutive lanes distinct 16-byte slots of a 128-byte window and every 16
// consecutive lanes distinct slots of a 256-byte window, so the reads are free
// of bank conflicts whether the LDS serves 8 lanes per cycle from 32 banks or
// 16 lanes per cycle from 64 banks.
#pragma once
#include <stddef.h>
#include <stdint.h>

#if defined(__HIPCC__)
#define CONVROT_HD __host__ __device__
#else
#define CONVROT_HD
#endif

namespace convrot {

constexpr int kTileRows = 32;     // rows per unit
constexpr int kTileK = 128;       // K per unit
constexpr int kUnitBytes = 2048;  // 32 rows x 128 codes / 2

CONVROT_HD inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// row r of a 32-row unit: bits (r1 ^ r2, r2 ^ r3)
CONVROT_HD inline int row_swizzle(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

// Bytes of the operand image of `rows` x K codes.
CONVROT_HD inline size_t image_bytes(int64_t rows, int64_t K)
{
    return (size_t)round_up(rows, kTileRows) * (size_t)round_up(K, kTileK) / 2;
}

// Byte offset of the 4-byte word holding the codes (row, k..k+7), k a
// multiple of 8: low nibbles are codes k..k+3, high nibbles k+4..k+7.
CONVROT_HD inline size_t image_word_offset(int64_t row, int64_t k, int64_t K_pad)
{
    const int64_t KB = K_pad / kTileK;
    const int64_t rt = row / kTileRows, r = row % kTileRows;
    const int64_t kb = k / kTileK, kl = k % kTileK;
    const int64_t ks = kl / 32, h = (kl % 32) / 16, d = (kl % 16) / 8;
    const int64_t ch = 2 * (ks / 2) + h;
    return (size_t)(rt * KB + kb) * kUnitBytes + (size_t)r * 64 + (size_t)((ch ^ row_swizzle((int)r)) * 16) +
           (size_t)((ks % 2) * 8 + d * 4);
}

// ---- FP6 operand image ------------------------------------------------------
// The same codes once more, as FP6 values for the FP6 matrix cores: OCP e2m3
// (sign, two exponent bits with bias 1, three mantissa bits) holds every
// integer in [-7, 7] exactly, and binary32 sums of their products are exact
// integers while below 2^24 (|dot| <= 49 K <= 802816).
//
//   unit (rt, kb) = rows [32 rt, 32 rt + 32) x k [128 kb, 128 kb + 128),
//   3072 bytes at ((rt * KB) + kb) * 3072; row r owns bytes [96 r, 96 r + 96).
//   The row is four 24-byte blocks: block b holds codes 32 b .. 32 b + 31, six
//   bits each, code 32 b + e at bit 6 e of the block read as one little-endian
//   bit string -- exactly the six registers one lane feeds to a 32x32x64 FP6
//   MFMA.  Block b is stored at block position b ^ row_swizzle6(r).
//
// Swizzle: a fragment is read as three 8-byte slots (0, 1, 2 of its block);
// each read has the lanes of a half wave read the same slot of the same
// logical block of 32 consecutive rows (96-byte stride).  Row r's block b
// sits at b ^ f(r), f(r) = 2 r3 + (r2 ^ r4) (bits of r).  In 8-byte units the
// slot addresses are 12 r + 3 (b ^ f(r)) + slot: modulo 16 (a 128-byte window)
// they differ for any 16 consecutive rows, because f tells apart the four rows
// of each residue r mod 4 (r2, r3 vary), and modulo 32 (a 256-byte window) for
// all 32 rows, because f tells apart the four rows of each residue r mod 8
// (r3, r4 vary): free of bank conflicts whether the LDS serves 16 lanes from
// 32 banks or 32 lanes from 64 banks per cycle.
constexpr int kUnit6Bytes = 3072;  // 32 rows x 128 codes x 6 bits
constexpr int kRow6Bytes = 96;

CONVROT_HD inline int row_swizzle6(int r) { return (((r >> 3) & 1) << 1) | (((r >> 2) ^ (r >> 4)) & 1); }

CONVROT_HD inline size_t image6_bytes(int64_t rows, int64_t K)
{
    return (size_t)round_up(rows, kTileRows) * (size_t)round_up(K, kTileK) * 3 / 4;
}

// Byte offset of logical byte b (0 .. 95) of row `row`, 128-K block kb.
CONVROT_HD inline size_t image6_byte_offset(int64_t row, int64_t kb, int b, int64_t K_pad)
{
    const int64_t KB = K_pad / kTileK;
    const int64_t rt = row / kTileRows, r = row % kTileRows;
    return (size_t)(rt * KB + kb) * kUnit6Bytes + (size_t)r * kRow6Bytes +
           (size_t)(((b / 24) ^ row_swizzle6((int)r)) * 24 + b % 24);
}

// OCP FP6 e2m3 bit pattern of an integer code in [-7, 7].
CONVROT_HD inline uint32_t fp6_e2m3(int q)
{
    const uint32_t mag = (uint32_t)(q < 0 ? -q : q);
    const uint32_t enc = (0xFEDCA840u >> (4 * mag)) & 0xFu;  // |q| = 0..7 -> 0, 4, 8, 10, 12, 13, 14, 15 (halved)
    return (q < 0 ? 0x20u : 0u) | (enc << 1);
}

// ---- flags carried by the group-size argument -------------------------------
// g is 64 or 256, optionally with these flags:
//   kRegularHadamard: rotate with the regular Hadamard matrix instead of the
//                     Sylvester one;
//   kInt4Image:       the weight image holds the INT4 codes only (0.5 bytes per
//                     weight), so every product runs on the INT8 matrix cores;
//                     without it the image also holds the FP6 copy (1.25 bytes
//                     per weight) that the FP6 block tile reads.
constexpr int kRegularHadamard = 0x10000;
constexpr int kInt4Image = 0x20000;
constexpr int kGroupFlags = kRegularHadamard | kInt4Image;
CONVROT_HD inline int group_size(int g) { return g & ~kGroupFlags; }
CONVROT_HD inline bool image_has_fp6(int g) { return (g & kInt4Image) == 0; }

// The weight image: the INT4 image of the N rows (read by the weight-streaming
// kernels and the INT8 block tiles), then, unless the image is INT4 only, the
// FP6 image of the same codes (read by the FP6 block tile).
CONVROT_HD inline size_t weight_image_bytes(int64_t N, int64_t K, bool fp6)
{
    return image_bytes(N, K) + (fp6 ? image6_bytes(N, K) : 0);
}
CONVROT_HD inline size_t weight_image6_offset(int64_t N, int64_t K) { return image_bytes(N, K); }

// Activations get an FP6 image too when the product goes to the block-tile
// GEMM (M > 32 rows) and the weight image has its FP6 copy.
CONVROT_HD inline bool act_has_fp6(int64_t M, bool fp6) { return fp6 && M > 32; }

// ---- rotation ---------------------------------------------------------------
// A row of K values is rotated as K rounded up to a whole number of groups,
// the missing values being zero; codes, scales and the product use that width.
CONVROT_HD inline int64_t rotated_width(int64_t K, int g)
{
    const int64_t gs = group_size(g);
    return (K + gs - 1) / gs * gs;
}

// ---- W4A16 -----------------------------------------------------------------
// The weight-only INT4 variant is the weight-bandwidth-bound regime: M <= 32.
constexpr int64_t kW4A16MaxRows = 32;

// The bf16 rotated rows are kept in the order in which the bf16 matrix-core
// product consumes them, so that every wave load is 1 KB of contiguous bytes:
// blocks of 16 rows, then 128-K units, then the four 32-K steps j of a unit,
// then the lane's quarter q of a step, then the 16 rows, each 16 bytes (8
// values).  Within unit kb the value at kl = k % 128 sits in step
// j = 2 b5 + b3 and quarter q = 2 b6 + b4 (b_i: bit i of kl), element kl % 8.
// Rows are rounded up to 16 and K to 128; the padding is never read.
CONVROT_HD inline size_t w16_rows_bytes(int64_t M, int64_t K)
{
    return (size_t)(round_up(M, 16) * round_up(K, kTileK) * 2);
}
// byte offset of the 16-byte word holding values k .. k+7 of row m (k % 8 == 0)
CONVROT_HD inline size_t w16_word_offset(int64_t m, int64_t k, int64_t K)
{
    const int64_t KB = (K + kTileK - 1) / kTileK;
    const int kl = (int)(k % kTileK);
    const int j = 2 * ((kl >> 5) & 1) + ((kl >> 3) & 1);
    const int q = 2 * ((kl >> 6) & 1) + ((kl >> 4) & 1);
    return (size_t)((((((m >> 4) * KB + k / kTileK) * 4 + j) * 4 + q) * 16 + (m & 15)) * 16);
}

// ---- GEMM plan -------------------------------------------------------------
// The GEMM covers the output with one of four block tiles.  Shapes 0 and 1
// run on the INT8 matrix cores from the INT4 image: shape 0 is 192 x 384,
// shape 1 is 192 x 192.  Shapes 2 and 3 run on the FP6 matrix cores from the
// FP6 image (twice the INT8 rate; bound by their LDS reads rather than by
// the matrix cores), the fastest per output where their tiles fill the chip:
// shape 2 is 256 x 256 with a three-stage ring, shape 3 is 192 x 384, whose
// 54 KB stages leave room for two (it fills the chip at 1536 x 12288).  The
// FP6 shapes are not candidates when the weight image is INT4 only.
// When there are too few tiles to fill the chip, the 192 x 192 tile's K range
// is split over S workgroups (the integer partial sums are exact in any
// order): S is the largest value <= 8 with S * tiles <= kSplitTargetWGs and
// >= 16 128-K blocks per split.  The plan never splits the other shapes;
// a plan given from outside (gemm_plan_forced, a test hook) may.  Of the
// shapes the plan takes the one with the smallest estimated time: rounds of
// workgroups x 128-K blocks per workgroup x tile area at gemm_shape_ns per
// 1024 outputs per block (measured on MI355X on the FLUX shapes), one
// prologue + epilogue (about 4 us) per round, and for a split the exchange of
// (S - 1) 4-byte partial tiles per tile through memory (written and read back
// at about 4 TB/s, plus 3 us).  M <= kStreamMaxRows goes to the
// weight-streaming kernel instead (one workgroup per 16 output columns, the
// activation codes of up to 128 rows read from L2 by every workgroup): at
// such M the block tiles leave most compute units idle.
constexpr int kSplitTargetWGs = 256;   // one workgroup per compute unit of an MI355X
constexpr int kSplitCounters = 256;    // counter slots: a split launch has at most this many tiles x splits
static_assert(kSplitTargetWGs <= kSplitCounters, "a plan's tiles x splits fit the counters");
constexpr int kMaxSplits = 8;
constexpr int kGemmShapes = 4;
constexpr int64_t kStreamMaxRows = 128;

CONVROT_HD constexpr int gemm_tile_m(int shape) { return shape == 2 ? 256 : 192; }
CONVROT_HD constexpr int gemm_tile_n(int shape) { return (shape == 0 || shape == 3) ? 384 : (shape == 1 ? 192 : 256); }
CONVROT_HD constexpr bool gemm_shape_fp6(int shape) { return shape >= 2; }
// nanoseconds per 1024 outputs per 128-K block, by shape (MI355X, FLUX shapes)
CONVROT_HD constexpr int gemm_shape_ns(int shape) { return shape == 0 ? 28 : (shape == 1 ? 30 : 19); }
// the shapes whose K range the plan splits
CONVROT_HD constexpr bool gemm_shape_splits(int shape) { return shape == 1; }
// threads of a block-tile workgroup, and bytes of its LDS stage ring
CONVROT_HD constexpr int gemm_threads(int shape) { return shape == 1 ? 256 : 512; }
CONVROT_HD constexpr int gemm_ring_bytes(int shape)
{
    return shape == 2   ? 3 * (256 / 32 + 256 / 32) * kUnit6Bytes
           : shape == 3 ? 2 * (192 / 32 + 384 / 32) * kUnit6Bytes
                        : 4 * (gemm_tile_m(shape) / 32 + gemm_tile_n(shape) / 32) * kUnitBytes;
}
// the block tile of (tile_m, tile_n), or -1; kTileFp6 or-ed into tile_n
// picks the FP6 tile where both kinds have that size (192 x 384)
constexpr int kTileFp6 = 0x10000;
CONVROT_HD constexpr int gemm_shape_of(int tile_m, int tile_n)
{
    return (tile_m == 192 && tile_n == 384)              ? 0
           : (tile_m == 192 && tile_n == 192)            ? 1
           : (tile_m == 256 && tile_n == 256)            ? 2
           : (tile_m == 256 && tile_n == (256 | kTileFp6)) ? 2
           : (tile_m == 192 && tile_n == (384 | kTileFp6)) ? 3
                                                         : -1;
}

struct GemmPlan {
    int shape;             // block tile shape (0 .. 2)
    int tiles_m, tiles_n;  // block tiles along M and N
    int splits;            // workgroups per tile along K
};

CONVROT_HD inline GemmPlan gemm_plan_forced(int64_t M, int64_t N, int shape, int splits)
{
    const int64_t bm = gemm_tile_m(shape), bn = gemm_tile_n(shape);
    return GemmPlan{shape, (int)((M + bm - 1) / bm), (int)((N + bn - 1) / bn), splits};
}

CONVROT_HD inline GemmPlan gemm_plan(int64_t M, int64_t N, int64_t K, bool fp6)
{
    GemmPlan best{0, 1, 1, 1};
    if (M <= kStreamMaxRows || N <= 0) return best;
    const int64_t KB = (K + kTileK - 1) / kTileK;
    int64_t best_ns = -1;
    for (int shape = 0; shape < kGemmShapes; ++shape) {
        if (gemm_shape_fp6(shape) && !fp6) continue;
        const int64_t bm = gemm_tile_m(shape), bn = gemm_tile_n(shape);
        const int64_t tm = (M + bm - 1) / bm, tn = (N + bn - 1) / bn;
        const int64_t tiles = tm * tn;
        int S = 1;
        while (gemm_shape_splits(shape) && S < kMaxSplits && (S + 1) * tiles <= kSplitTargetWGs && KB / (S + 1) >= 16)
            ++S;
        const int64_t rounds = (tiles * S + kSplitTargetWGs - 1) / kSplitTargetWGs;
        int64_t ns = rounds * ((KB + S - 1) / S) * (bm * bn / 1024) * gemm_shape_ns(shape) + rounds * 4000;
        if (S > 1) ns += tiles * (S - 1) * bm * bn * 8 / 4000 + 3000;
        if (best_ns < 0 || ns < best_ns) {
            best_ns = ns;
            best = GemmPlan{shape, (int)tm, (int)tn, S};
        }
    }
    return best;
}

// ---- split-K exchange geometry -----------------------------------------------
// The tile's 4-byte sums are exchanged in S sub-blocks.  A wave owns BI x BJ
// MFMA tiles of 32 x 32 ("pairs"); pair (j, i) has row-major number
// r = i BJ + j, and sub-block b holds the pairs with r in [first(b),
// first(b + 1)), first(b) = ceil(b P / S) for P = BI BJ pairs: contiguous
// runs, so that whole 32-row blocks of Y go to one workgroup where S allows.
// For each sub-block, the S - 1 first workgroups (tickets) of a split tile
// store their partial sums of it into slot `ticket` of the tile's partial
// area; the last one copies the sub-block's part of every slot into its LDS
// ring, pair by pair, and adds it.  Slot (tile, ticket) is slot number
// tile (S - 1) + ticket; inside it, 8-byte word u of thread t sits at
// (u threads + t) 8, so that one store instruction of a wave covers 512
// contiguous bytes; pair (j, i) holds words 8 p .. 8 p + 7, p = j BI + i, of
// every thread, one contiguous run.  Sub-block b of tile `tile` has its own
// two counters (tickets, finished writers): counter words split_counter and
// split_counter + kSplitCounters.  The kernels and the host-side footprint
// check (convrot_split_k_extent) address all of this through these functions
// only.
CONVROT_HD constexpr int gemm_wave_tiles_m(int shape) { return shape == 2 ? 4 : 3; }  // BI
CONVROT_HD constexpr int gemm_wave_tiles_n(int shape) { return shape == 2 ? 2 : 3; }  // BJ
CONVROT_HD constexpr int split_pairs(int shape) { return gemm_wave_tiles_m(shape) * gemm_wave_tiles_n(shape); }
CONVROT_HD constexpr int split_sub_first(int shape, int splits, int sub)
{
    return (sub * split_pairs(shape) + splits - 1) / splits;
}
CONVROT_HD constexpr int split_sub_of(int shape, int splits, int i, int j)
{
    return (i * gemm_wave_tiles_n(shape) + j) * splits / split_pairs(shape);
}
// slot pair index p = j BI + i of row-major pair number r
CONVROT_HD constexpr int split_pair_of(int shape, int r)
{
    return (r % gemm_wave_tiles_n(shape)) * gemm_wave_tiles_m(shape) + r / gemm_wave_tiles_n(shape);
}
CONVROT_HD constexpr size_t split_slot_bytes(int shape) { return (size_t)gemm_tile_m(shape) * gemm_tile_n(shape) * 4; }
CONVROT_HD constexpr int split_words_per_thread(int shape)
{
    return (int)(split_slot_bytes(shape) / 8 / gemm_threads(shape));
}
CONVROT_HD inline size_t split_store_offset(int shape, int tile, int splits, int ticket, int word, int thread)
{
    return ((size_t)tile * (splits - 1) + ticket) * split_slot_bytes(shape) +
           ((size_t)word * gemm_threads(shape) + thread) * 8;
}
// bytes of one pair's sums in a slot, and how many pairs the LDS ring holds
CONVROT_HD constexpr int split_pair_bytes(int shape) { return 8 * gemm_threads(shape) * 8; }
CONVROT_HD constexpr int split_pairs_per_copy(int shape) { return gemm_ring_bytes(shape) / split_pair_bytes(shape); }
// 16-byte piece `lane` of 1 KB chunk `chunk` of pair `pair` of slot `slot`
CONVROT_HD inline size_t split_copy_offset(int shape, int tile, int splits, int slot, int pair, int chunk, int lane)
{
    return split_store_offset(shape, tile, splits, slot, 8 * pair, 0) + (size_t)chunk * 1024 + (size_t)lane * 16;
}
CONVROT_HD constexpr int split_counter(int tile, int splits, int sub) { return tile * splits + sub; }
// The workspace's status word (at a fixed offset, cleared by every activation
// step): kStatusSplitTimeout when a split-K finalizer stopped waiting.
constexpr uint32_t kStatusSplitTimeout = 1;
constexpr int kSplitSpinLimit = 1 << 26;  // sleeps of 128 clocks: seconds, far beyond any real wait

// Bytes of split-K partial tiles of a plan: (S - 1) slots per tile.
CONVROT_HD inline size_t gemm_partial_bytes(const GemmPlan& p)
{
    if (p.splits <= 1) return 0;
    return (size_t)p.tiles_m * p.tiles_n * (size_t)(p.splits - 1) * split_slot_bytes(p.shape);
}

// ---- single-kernel linear ---------------------------------------------------
// convrot_linear is one kernel (small_m_kernel) when M <= 4 and an activation
// row is one to four whole waves of the prep (K / P lanes, P = 16 for g = 256,
// 8 for g = 64); otherwise an activation kernel followed by the GEMM.
constexpr int kSmallRows = 4;
CONVROT_HD inline bool single_kernel_linear(int64_t M, int64_t K, int g)
{
    const int64_t lanes = round_up(K, kTileK) / (group_size(g) == 256 ? 16 : 8);
    return M >= 1 && M <= kSmallRows && lanes >= 64 && lanes <= 256;
}

}  // namespace convrot
