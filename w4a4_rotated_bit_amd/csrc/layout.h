// layout.h -- byte layouts of the ConvRot W4A4 operands in device memory.
//
// Two "images" are laid out so that the GEMM moves them with straight 16-byte
// copies (global memory -> LDS) and reads MFMA fragments out of LDS without
// bank conflicts.  Both are tiled in 32-row/column by 128-K units; every unit
// is contiguous, and the units of one 32-row (or 32-column) strip are
// consecutive along K, so a strip streams linearly.
//
// Activation image (signed INT8 codes, one byte per code):
//   unit (mt, kb) = rows [32 mt, 32 mt + 32) x k [128 kb, 128 kb + 128),
//   4096 bytes at ((mt * KB) + kb) * 4096, KB = K_pad / 128.
//   Row r of the unit owns bytes [128 r, 128 r + 128): eight 16-byte chunks;
//   logical chunk c holds codes k = 128 kb + 16 c + (0..15) in natural order
//   and is stored at chunk position c ^ act_swizzle(r).
//
// Weight image (signed INT4 codes, two per byte):
//   unit (nt, kb) = columns [32 nt, 32 nt + 32) x k [128 kb, 128 kb + 128),
//   2048 bytes at ((nt * KB) + kb) * 2048.
//   Column c owns bytes [64 c, 64 c + 64): four 16-byte chunks; logical chunk
//   ch = 2 p + h (p = pair of 32-wide k-steps, h = half of a k-step) is
//   stored at chunk position ch ^ wgt_swizzle(c) and holds
//     bytes 0..7 : k-step 2p,   codes k = 32(2p)   + 16h + t, t = 0..15
//     bytes 8..15: k-step 2p+1, codes k = 32(2p+1) + 16h + t, t = 0..15
//   Within each 8-byte group, dword d (0..1) byte b (0..3) holds code
//   t = 8d + b in its low nibble and code t = 8d + 4 + b in its high nibble,
//   so that (dword << 4) & 0xF0F0F0F0 and dword & 0xF0F0F0F0 are the codes
//   t = 8d + (0..3) and 8d + (4..7) as INT8 values times 16, in natural order.
//
// Padding: rows (columns) up to a multiple of 32 and K up to a multiple of
// 128 are stored as code 0.
//
// Swizzles: an MFMA fragment read (ds_read_b128) has the 32 lanes of one half
// wave read the same logical chunk of 32 consecutive rows (columns).  The
// swizzles give every 8 consecutive lanes distinct 16-byte slots of a 128-byte
// window and every 16 consecutive lanes distinct slots of a 256-byte window,
// so the reads are free of bank conflicts whether the LDS serves 8 lanes per
// cycle from 32 banks or 16 lanes per cycle from 64 banks.
#pragma once
#include <stddef.h>
#include <stdint.h>

#if defined(__HIPCC__)
#define CONVROT_HD __host__ __device__
#else
#define CONVROT_HD
#endif

namespace convrot {

constexpr int kTileRows = 32;     // rows (or columns) per unit
constexpr int kTileK = 128;       // K per unit
constexpr int kActUnitBytes = 4096;
constexpr int kWgtUnitBytes = 2048;

CONVROT_HD inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// row r of a 32-row unit: bits (r0 ^ r3, r1, r2)
CONVROT_HD inline int act_swizzle(int r) { return (r ^ (r >> 3)) & 7; }
// column c of a 32-column unit: bits (c1 ^ c2, c2 ^ c3)
CONVROT_HD inline int wgt_swizzle(int c) { return ((c >> 1) ^ (c >> 2)) & 3; }

// Byte offset of the 16-byte chunk holding activation codes (row m, k..k+15),
// k a multiple of 16.
CONVROT_HD inline size_t act_chunk_offset(int64_t m, int64_t k, int64_t K_pad)
{
    const int64_t KB = K_pad / kTileK;
    const int64_t mt = m / kTileRows, r = m % kTileRows;
    const int64_t kb = k / kTileK, c = (k % kTileK) / 16;
    return (size_t)(mt * KB + kb) * kActUnitBytes + (size_t)r * 128 + (size_t)((c ^ act_swizzle((int)r)) * 16);
}

// Byte offset of the 4-byte word holding weight codes (column n, k..k+7),
// k a multiple of 8: low nibbles are codes k..k+3, high nibbles k+4..k+7.
CONVROT_HD inline size_t wgt_word_offset(int64_t n, int64_t k, int64_t K_pad)
{
    const int64_t KB = K_pad / kTileK;
    const int64_t nt = n / kTileRows, c = n % kTileRows;
    const int64_t kb = k / kTileK, kl = k % kTileK;
    const int64_t ks = kl / 32, h = (kl % 32) / 16, d = (kl % 16) / 8;
    const int64_t ch = 2 * (ks / 2) + h;
    return (size_t)(nt * KB + kb) * kWgtUnitBytes + (size_t)c * 64 + (size_t)((ch ^ wgt_swizzle((int)c)) * 16) +
           (size_t)((ks % 2) * 8 + d * 4);
}

}  // namespace convrot
