"""Comparison rules between the HIP path and the CPU oracle.

Codes: bit-exact, except that an element whose oracle value r/s lies within
1e-4 of a rounding tie (|frac(|r/s|) - 0.5| < 1e-4) may differ by +-1; such
mismatches are counted and may not exceed 1e-5 of the elements.
Scales: bit-exact.  int32 sums: bit-exact.  Rotated values: within 1e-5 of
the row absmax.  Y (bf16): bit-exact when every code and scale matched;
otherwise max|dY| <= 1e-2 * max|Y| and bit-exact on rows whose codes all
matched.
"""
import numpy as np

TIE_BAND = 1e-4
MISMATCH_FRACTION = 1e-5


def w16_word_index(M: int, Kr: int) -> np.ndarray:
    """Index of the 16-byte word (8 bf16 values) holding rotated values
    k .. k + 7 of row m in a W4A16 workspace, as [M][Kr / 8], by the layout
    include/convrot.h states for it: words ordered by 16-row block, 128-K
    unit, step j, quarter q, row.  The GPU tests read the kernel's output
    through it (so a kernel that wrote elsewhere would fail them) and a CPU
    test checks that it is one-to-one inside the size the query returns."""
    KB = -(-Kr // 128)
    m = np.arange(M)[:, None]
    k = np.arange(0, Kr, 8)[None, :]
    kl = k % 128
    j = 2 * ((kl >> 5) & 1) + ((kl >> 3) & 1)
    q = 2 * ((kl >> 6) & 1) + ((kl >> 4) & 1)
    return ((((m // 16) * KB + k // 128) * 4 + j) * 4 + q) * 16 + m % 16


def bf16_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def compare_codes(gpu_q, ora_q, ora_r, ora_s, what="codes"):
    """Returns the number of (allowed) tie-band mismatches; raises AssertionError
    on any other difference."""
    gq = np.asarray(gpu_q).astype(np.int64)
    oq = np.asarray(ora_q).astype(np.int64)
    assert gq.shape == oq.shape, (what, gq.shape, oq.shape)
    diff = gq - oq
    bad = np.argwhere(diff != 0)
    if bad.size == 0:
        return 0
    r = np.asarray(ora_r, dtype=np.float64)
    s = np.asarray(ora_s, dtype=np.float64)
    rows, cols = bad[:, 0], bad[:, 1]
    ratio = np.abs(r[rows, cols] / s[rows])
    tie_dist = np.abs(ratio - np.floor(ratio) - 0.5)
    outside = (tie_dist >= TIE_BAND) | (np.abs(diff[rows, cols]) > 1)
    assert not outside.any(), f"{what}: {int(outside.sum())} mismatches outside the tie band, e.g. " \
                              f"{bad[outside][:5].tolist()}"
    assert len(bad) <= MISMATCH_FRACTION * gq.size, f"{what}: {len(bad)} tie-band mismatches in {gq.size}"
    return len(bad)


def compare_rotated(gpu_r, ora_r):
    g = np.asarray(gpu_r, dtype=np.float64)
    o = np.asarray(ora_r, dtype=np.float64)
    amax = np.abs(o).max(axis=1, keepdims=True)
    err = np.abs(g - o)
    assert np.all(err <= 1e-5 * amax + 0.0), f"rotated values: max err/absmax {float((err / np.maximum(amax, 1e-30)).max())}"
    return int(np.count_nonzero(g != o))


def compare_y(gpu_y, ora_y, codes_equal_rows=None):
    """gpu_y / ora_y: bf16 bits.  codes_equal_rows: bool per row, True where the
    row's activation codes (and all weight codes involved) matched."""
    gy = np.asarray(gpu_y, dtype=np.uint16)
    oy = np.asarray(ora_y, dtype=np.uint16)
    assert gy.shape == oy.shape
    if codes_equal_rows is None or np.all(codes_equal_rows):
        n_diff = int(np.count_nonzero(gy != oy))
        assert n_diff == 0, f"Y differs in {n_diff} of {gy.size} elements although every code matched"
        return 0
    gf, of = bf16_to_f64(gy), bf16_to_f64(oy)
    rel = np.abs(gf - of).max() / max(np.abs(of).max(), 1e-30)
    assert rel <= 1e-2, f"max |dY| / max |Y| = {rel}"
    rows = np.asarray(codes_equal_rows)
    assert np.array_equal(gy[rows], oy[rows])
    return int(np.count_nonzero(gy != oy))
