"""Host-side checks of the C ABI, runnable without a GPU: the library loads and
exports every function include/convrot.h declares; sizes, argument checks and
status codes; the host layout tools against the oracle's packing (convrot-mlx
README, "What is included": reversible N x packed-K and K x packed-N layouts).
No device entry point is called here."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from w4a4_rotated_bit_amd import binding as B

from ._parity import w16_word_index

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "convrot.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(convrot_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = B.load()
    names = _declared_functions()
    assert len(names) >= 20
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    # and the binding knows the signature of each one
    assert set(names) == set(B._SIGNATURES), set(names) ^ set(B._SIGNATURES)


def test_workspace_image_offset_matches_header():
    m = re.search(r"#define\s+CONVROT_WORKSPACE_IMAGE_OFFSET\s+(\d+)", open(HEADER).read())
    assert m and int(m.group(1)) == B.WORKSPACE_IMAGE_OFFSET


def test_regular_flag_matches_header():
    m = re.search(r"#define\s+CONVROT_REGULAR_HADAMARD\s+(0x[0-9a-fA-F]+)", open(HEADER).read())
    assert m and int(m.group(1), 16) == B.CONVROT_REGULAR_HADAMARD


def test_matrix_core_probe_constants_and_argument_checks():
    """The probe kinds match the header, and bad arguments are refused before
    any device call (so the check runs without a GPU)."""
    import ctypes
    text = open(HEADER).read()
    for name in ("CONVROT_PROBE_FP6", "CONVROT_PROBE_INT8"):
        m = re.search(rf"#define\s+{name}\s+(\d+)", text)
        assert m and int(m.group(1)) == getattr(B, name)
    lib = B.load()
    count = ctypes.c_int64(0)
    buf = ctypes.create_string_buffer(16)
    for kind, iters in ((0, 10), (3, 10), (B.CONVROT_PROBE_FP6, 0), (B.CONVROT_PROBE_INT8, (1 << 24) + 1)):
        rc = lib.convrot_matrix_core_probe(kind, iters, ctypes.cast(buf, ctypes.c_void_p), 16, ctypes.byref(count), None)
        assert rc == B.CONVROT_EINVAL, (kind, iters, rc)
    assert lib.convrot_matrix_core_probe(1, 10, None, 16, ctypes.byref(count), None) == B.CONVROT_EINVAL
    assert lib.convrot_matrix_core_probe(1, 10, ctypes.cast(buf, ctypes.c_void_p), 16, None, None) == B.CONVROT_EINVAL


def test_image_flag_status_word_and_test_flag_match_header():
    text = open(HEADER).read()
    m = re.search(r"#define\s+CONVROT_INT4_IMAGE\s+(0x[0-9a-fA-F]+)", text)
    assert m and int(m.group(1), 16) == B.CONVROT_INT4_IMAGE
    for name, value in (("CONVROT_WORKSPACE_STATUS_OFFSET", B.WORKSPACE_STATUS_OFFSET),
                        ("CONVROT_STATUS_SPLIT_TIMEOUT", B.CONVROT_STATUS_SPLIT_TIMEOUT),
                        ("CONVROT_TEST_SPLIT_TIMEOUT", B.CONVROT_TEST_SPLIT_TIMEOUT)):
        m = re.search(r"#define\s+%s\s+(\d+)" % name, text)
        assert m and int(m.group(1)) == value, name
    # the status word sits right after the 512 counters, before the activation image
    assert B.WORKSPACE_STATUS_OFFSET == 512 * 4 < B.WORKSPACE_IMAGE_OFFSET


def test_mfma_kinds_match_header():
    text = open(HEADER).read()
    for name in ("CONVROT_MFMA_I8", "CONVROT_MFMA_FP6"):
        m = re.search(r"#define\s+%s\s+(\d+)" % name, text)
        assert m and int(m.group(1)) == getattr(B, name)


def test_version_and_status_strings():
    assert B.convrot_version().startswith("convrot-gfx950")
    for code in (0, 1, 2, 3, 4):
        assert B.convrot_status_string(code)
    assert B.convrot_status_string(99) == "unknown status"


def _int4_plane(rows, K):
    """Bytes of the INT4 part of a weight image (rows padded to 32, K to 128)."""
    return -(-rows // 32) * 32 * (-(-K // 128) * 128) // 2


@pytest.mark.parametrize("N,K,g,int4", [
    (1024, 1024, 256, 1024 * 1024 // 2),
    (9216, 3072, 256, 9216 * 3072 // 2),
    (33, 192, 64, 64 * 256 // 2),        # N padded to 64, K to 256
])
def test_weight_image_bytes(N, K, g, int4):
    # the INT4 codes, then the same codes as FP6 (six bits each)
    assert _int4_plane(N, K) == int4
    assert B.convrot_weight_image_bytes(N, K, g) == int4 + int4 * 3 // 2
    # INT4 only: half a byte per (padded) weight, with either rotation
    assert B.convrot_weight_image_bytes(N, K, g | B.CONVROT_INT4_IMAGE) == int4
    assert B.convrot_weight_image_bytes(N, K, g | B.CONVROT_INT4_IMAGE | B.CONVROT_REGULAR_HADAMARD) == int4


def test_plan_of_the_flux_shapes():
    """The block tile each FLUX-shaped linear gets (measured choices on MI355X:
    the FP6 256 x 256 tile where its tiles fill one round, the FP6 192 x 384
    tile where 256 x 256 would need two rounds and 192 x 384 fills the chip
    exactly, the split 192 x 192 INT8 tile for the long reduction of the
    down-projection)."""
    FP6, I8 = B.CONVROT_MFMA_FP6, B.CONVROT_MFMA_I8
    assert B.convrot_linear_plan(1536, 3072, 9216, 256) == {"mfma": FP6, "tile": (256, 256), "splits": 1}
    assert B.convrot_linear_plan(4096, 3072, 3072, 256) == {"mfma": FP6, "tile": (256, 256), "splits": 1}
    assert B.convrot_linear_plan(1536, 3072, 12288, 256) == {"mfma": FP6, "tile": (192, 384), "splits": 1}
    assert B.convrot_linear_plan(1536, 12288, 3072, 256) == {"mfma": I8, "tile": (192, 192), "splits": 2}
    assert B.convrot_linear_plan(16, 3072, 12288, 256) == {"mfma": I8, "tile": (0, 0), "splits": 1}
    # up to 128 rows the weight is streamed; from 129 on, block tiles
    assert B.convrot_linear_plan(64, 1024, 1024, 256) == {"mfma": I8, "tile": (0, 0), "splits": 1}
    assert B.convrot_linear_plan(128, 2048, 2048, 64) == {"mfma": I8, "tile": (0, 0), "splits": 1}
    assert B.convrot_linear_plan(129, 2048, 2048, 64)["tile"] != (0, 0)
    assert B.convrot_linear_plan(0, 3072, 12288, 256) == {"mfma": 0, "tile": (0, 0), "splits": 1}
    # only the 192 x 192 tile is ever split
    for M, N, K in [(256, 3072, 16384), (1024, 1024, 8192), (300, 9000, 12288), (64, 64, 16384)]:
        p = B.convrot_linear_plan(M, K, N, 256)
        assert p["splits"] == 1 or p["tile"] == (192, 192), (M, N, K, p)
    with pytest.raises(B.ConvRotError):
        B.convrot_linear_plan(64, 1001, 64, 256)


def test_plan_of_the_flux_shapes_with_an_int4_image():
    """Without the FP6 copy every product runs on the INT8 matrix cores: the
    QKV and stress shapes move to INT8 block tiles, the others keep theirs."""
    I8, F = B.CONVROT_MFMA_I8, B.CONVROT_INT4_IMAGE
    assert B.convrot_linear_plan(1536, 3072, 9216, 256 | F) == {"mfma": I8, "tile": (192, 384), "splits": 1}
    assert B.convrot_linear_plan(1536, 3072, 12288, 256 | F) == {"mfma": I8, "tile": (192, 384), "splits": 1}
    assert B.convrot_linear_plan(1536, 12288, 3072, 256 | F) == {"mfma": I8, "tile": (192, 192), "splits": 2}
    for M, N, K in [(4096, 3072, 3072), (64, 1024, 1024), (128, 2048, 2048), (300, 9000, 12288)]:
        assert B.convrot_linear_plan(M, K, N, 256 | F)["mfma"] == I8, (M, N, K)


def test_workspace_bytes():
    # 512 counters (2048 B) and the status word, the activation INT4 image at 4096
    # (M up to 32 rows, K up to 128) | the same codes as FP6 when M > 32 (3/4 byte
    # each) | sx | split-K partials, each part 256-byte aligned (values worked out
    # by hand from that layout)
    # M <= 32: weight streaming, never split, no FP6 image
    assert B.convrot_workspace_bytes(1, 3072, 12288, 256) == 4096 + 49152 + 256
    # 1536 x 3072 -> 9216: 216 FP6 tiles of 256 x 256 fill the GPU, no split
    assert B.convrot_workspace_bytes(1536, 3072, 9216, 256) == 4096 + 2359296 + 3538944 + 6144
    # 1536 x 12288 -> 3072: 128 tiles of 192 x 192, K split 2 ways -> 1 partial tile of
    # 192 x 192 4-byte sums per tile (fewer partial bytes than 72 tiles of 256 x 256
    # split 3 ways)
    assert B.convrot_workspace_bytes(1536, 12288, 3072, 256) == 4096 + 9437184 + 14155776 + 6144 + 128 * 147456
    # 1536 x 3072 -> 12288: 288 tiles of 256 x 256 would take two rounds; 256 tiles
    # of 192 x 384 take one, unsplit
    assert B.convrot_workspace_bytes(1536, 3072, 12288, 256) == 4096 + 2359296 + 3538944 + 6144
    # 4096 x 3072 -> 3072: 192 FP6 tiles of 256 x 256, unsplit
    assert B.convrot_workspace_bytes(4096, 3072, 3072, 256) == 4096 + 6291456 + 9437184 + 16384
    # 256 x 4096 -> 256: 2 x 2 tiles of 192 x 192; 32 K blocks split 2 ways (at least
    # 16 K blocks per split) -> 1 partial tile each
    assert B.convrot_workspace_bytes(256, 4096, 256, 256) == 4096 + 524288 + 786432 + 1024 + 4 * 147456
    # 5 x 192 -> N: M <= 32
    assert B.convrot_workspace_bytes(5, 192, 100, 64) == 4096 + 32 * 256 // 2 + 256
    # K not a multiple of g: sizes follow the rotated width (1000 -> 1024)
    assert B.convrot_workspace_bytes(64, 1000, 1024, 256) == B.convrot_workspace_bytes(64, 1024, 1024, 256)
    assert B.convrot_weight_image_bytes(100, 328, 256) == 128 * 512 // 2 * 5 // 2
    # N = 0: nothing to split
    assert B.convrot_workspace_bytes(1536, 12288, 0, 256) == 4096 + 9437184 + 14155776 + 6144
    # INT4 image: no FP6 activation part; QKV on 192 x 384 unsplit, the
    # down-projection on 192 x 192 split 2 ways as before
    F = B.CONVROT_INT4_IMAGE
    assert B.convrot_workspace_bytes(1536, 3072, 9216, 256 | F) == 4096 + 2359296 + 6144
    assert B.convrot_workspace_bytes(1536, 12288, 3072, 256 | F) == 4096 + 9437184 + 6144 + 128 * 147456


def _ceil(a, b):
    return -(-a // b)


_F6 = B.CONVROT_TILE_FP6
_RING = {(192, 384): 4 * 18 * 2048, (192, 192): 4 * 12 * 2048, (256, 256): 3 * 16 * 3072,
         (192, 384 | _F6): 2 * 18 * 3072}


@pytest.mark.parametrize("M,K,N", [(1536, 12288, 3072), (1500, 12000, 3000), (256, 4096, 256), (64, 16384, 64)])
@pytest.mark.parametrize("tile", [(192, 384), (192, 192), (256, 256), (192, 384 | _F6)])
@pytest.mark.parametrize("splits", [1, 2, 3, 4, 8])
def test_split_k_exchange_stays_inside_its_workspace(M, K, N, tile, splits):
    """Every address of the split-K exchange, enumerated on the host through the
    kernels' own address functions: the partial-tile stores and copies end
    exactly at (S - 1) slots per tile, which is the room the same plan's
    workspace size sets aside after its other parts; the two counters of every
    (tile, sub-block) stay in the 512 counter words, and the finalizer's
    copies of a sub-block's pairs stay in the LDS ring."""
    tm, tn = tile[0], tile[1] & ~_F6
    tiles = _ceil(M, tm) * _ceil(N, tn)
    if splits > 1 and tiles * splits > 256:
        with pytest.raises(B.ConvRotError):
            B.convrot_split_k_extent(M, K, N, tile, splits)
        return
    ext = B.convrot_split_k_extent(M, K, N, tile, splits)
    slot = tm * tn * 4
    assert ext["partial_end"] == tiles * (splits - 1) * slot
    ws = B.convrot_workspace_bytes_tiled(M, K, N, tile, splits)
    assert ws - B.convrot_workspace_bytes_tiled(M, K, N, tile, 1) == ext["partial_end"]
    if splits > 1:
        assert ext["counters_used"] == 256 + tiles * splits <= 512
        threads = 256 if tile == (192, 192) else 512
        pair = 64 * threads                      # one MFMA tile's sums of every thread
        pairs = slot // pair                     # MFMA tiles per wave
        most = -(-pairs // splits)               # pairs of the largest sub-block
        assert ext["lds_end"] == min(most, _RING[tile] // pair) * pair <= _RING[tile]
    else:
        assert ext == {"partial_end": 0, "counters_used": 0, "lds_end": 0}


def test_split_k_fault_reading():
    """The down-projection shape, with the block tiles and splits that a timing
    probe once forced when the GPU faulted (192 x 384 split 4 ways, 256 x 256
    split 3 ways): their exchange needs 56.6 MB and 37.7 MB of partial tiles,
    while a workspace sized by the library's own plan for this shape (192 x 192
    split 2 ways) has 18.9 MB of room -- a forced launch given such a workspace
    writes tens of MB past its end.  The plan's own split fits exactly."""
    M, K, N = 1536, 12288, 3072
    room = B.convrot_workspace_bytes(M, K, N, 256) - B.convrot_workspace_bytes_tiled(M, K, N, (256, 256), 1)
    assert room == 128 * 192 * 192 * 4 == 18874368
    assert B.convrot_split_k_extent(M, K, N, (192, 192), 2)["partial_end"] == room
    e4 = B.convrot_split_k_extent(M, K, N, (192, 384), 4)["partial_end"]
    e3 = B.convrot_split_k_extent(M, K, N, (256, 256), 3)["partial_end"]
    assert e4 == 64 * 3 * 192 * 384 * 4 == 56623104 and e4 - room == 37748736
    assert e3 == 72 * 2 * 256 * 256 * 4 == 37748736 and e3 - room == 18874368


def _gemm_i32_tiled_status(M, K, N, tile, splits, ws_bytes, flags=0):
    lib = B.load()
    p = ctypes.c_void_p(1 << 20)   # aligned, never dereferenced: the checks come first
    return lib.convrot_gemm_i32_tiled(p, M, K, p, N, p, tile[0], tile[1], splits, flags, p, ws_bytes, None)


def test_gemm_i32_tiled_checks():
    M, K, N = 1536, 12288, 3072
    need = B.convrot_workspace_bytes_tiled(M, K, N, (256, 256), 3)
    assert _gemm_i32_tiled_status(M, K, N, (256, 256), 3, need - 1) == B.CONVROT_EWORKSPACE
    # the plan-sized workspace is too small for the forced split
    assert _gemm_i32_tiled_status(M, K, N, (256, 256), 3, B.convrot_workspace_bytes(M, K, N, 256)) == \
        B.CONVROT_EWORKSPACE
    F6 = B.CONVROT_TILE_FP6
    for tile, splits in [((128, 128), 1), ((192, 384), 0), ((192, 384), 9), ((256, 256), -1), ((192, 192 | F6), 1),
                         ((192 | F6, 384), 1), ((192, 384 | F6 | 1), 1)]:
        assert _gemm_i32_tiled_status(M, K, N, tile, splits, 1 << 40) == B.CONVROT_EINVAL, (tile, splits)
    assert _gemm_i32_tiled_status(32, K, N, (192, 192), 1, 1 << 40) == B.CONVROT_EINVAL       # M <= 32
    assert _gemm_i32_tiled_status(M, 256, N, (192, 192), 3, 1 << 40) == B.CONVROT_EINVAL      # S > K blocks
    assert _gemm_i32_tiled_status(4096, K, 9216, (192, 192), 2, 1 << 40) == B.CONVROT_EINVAL  # > 256 tiles split
    assert _gemm_i32_tiled_status(M, K, N, (192, 192), 2, 1 << 40, flags=2) == B.CONVROT_EINVAL
    with pytest.raises(B.ConvRotError):
        B.convrot_workspace_bytes_tiled(M, K, N, (192, 96), 1)
    # the FP6 192 x 384 tile reads the FP6 copy of the codes, so its workspace
    # holds the FP6 activation image the INT8 tile of the same size does not
    fp6_part = B.convrot_workspace_bytes_tiled(M, K, N, (192, 384 | F6), 1) - \
        B.convrot_workspace_bytes_tiled(M, K, N, (192, 384), 1)
    assert fp6_part >= M * K * 3 // 4
    assert B.convrot_workspace_bytes_tiled(M, K, N, (256, 256 | F6), 1) == \
        B.convrot_workspace_bytes_tiled(M, K, N, (256, 256), 1)


@pytest.mark.parametrize("M,K,N,g,want", [(1, 3072, 12288, 256, 1), (4, 4096, 64, 256, 1), (5, 3072, 64, 256, 2),
                                          (1, 768, 64, 256, 2), (1, 4352, 64, 256, 2), (4, 512, 64, 64, 1),
                                          (4, 2176, 64, 64, 2), (1536, 3072, 9216, 256, 2), (0, 3072, 64, 256, 0),
                                          (3, 3072, 0, 256, 0)])
def test_linear_kernel_count(M, K, N, g, want):
    # one kernel when M <= 4 and a row is 1..4 whole waves of the prep (K / 16 lanes for g = 256, K / 8 for g = 64)
    assert B.convrot_linear_kernel_count(M, K, N, g) == want


@pytest.mark.parametrize("N,K,g", [(16, 100, 64), (16, 512, 128), (16, 0, 64), (-1, 256, 256), (16, 32768, 256)])
def test_size_queries_reject_bad_shapes(N, K, g):
    with pytest.raises(B.ConvRotError) as e:
        B.convrot_weight_image_bytes(N, K, g)
    assert e.value.status == B.CONVROT_EINVAL


def _validate_linear(**over):
    args = dict(X=4096, M=64, K=1024, image=8192, sw=16384, bias=0, N=1024, g=256, Y=32768, ws=65536,
                ws_bytes=B.convrot_workspace_bytes(64, 1024, 1024, 256))
    args.update(over)
    return B.convrot_validate_linear(args["X"], args["M"], args["K"], args["image"], args["sw"], args["bias"],
                                     args["N"], args["g"], args["Y"], args["ws"], args["ws_bytes"])


def test_validate_linear_statuses():
    assert _validate_linear() == B.CONVROT_OK
    assert _validate_linear(bias=2) == B.CONVROT_OK
    assert _validate_linear(g=128) == B.CONVROT_EINVAL
    R = B.CONVROT_REGULAR_HADAMARD
    assert _validate_linear(g=256 | R) == B.CONVROT_OK
    assert _validate_linear(g=64 | R) == B.CONVROT_OK
    assert _validate_linear(g=128 | R) == B.CONVROT_EINVAL
    assert _validate_linear(g=256 | (R << 2)) == B.CONVROT_EINVAL    # unknown flag
    assert _validate_linear(g=256 | B.CONVROT_INT4_IMAGE | R) == B.CONVROT_OK
    assert _validate_linear(g=R) == B.CONVROT_EINVAL
    assert _validate_linear(K=1000) == B.CONVROT_OK               # last group zero-padded to 1024
    assert _validate_linear(K=1004) == B.CONVROT_EINVAL           # rows are whole 16-byte runs
    assert _validate_linear(K=16392) == B.CONVROT_EINVAL          # rotated width above the maximum
    assert _validate_linear(X=0) == B.CONVROT_EINVAL
    assert _validate_linear(Y=0) == B.CONVROT_EINVAL
    assert _validate_linear(image=0) == B.CONVROT_EINVAL
    assert _validate_linear(X=4100) == B.CONVROT_EINVAL           # misaligned
    assert _validate_linear(sw=16386) == B.CONVROT_EINVAL         # misaligned
    assert _validate_linear(bias=3) == B.CONVROT_EINVAL           # misaligned
    assert _validate_linear(ws_bytes=1000) == B.CONVROT_EWORKSPACE
    assert _validate_linear(M=0, X=0, Y=0) == B.CONVROT_OK        # empty input is a no-op
    assert _validate_linear(N=0) == B.CONVROT_OK
    assert _validate_linear(M=-1) == B.CONVROT_EINVAL


def test_w4a16_row_layout_fits_the_workspace():
    """The bf16 row layout that include/convrot.h states for the W4A16
    workspace (16-byte words ordered by 16-row block, 128-K unit, step j,
    quarter q, row) places every 8-value word of every row at a distinct word
    inside the size the query returns, for ragged M and for K_rot % 128 == 64."""
    for M, K, g in [(1, 3072, 256), (5, 192, 64), (17, 1000, 256), (32, 2048, 256), (31, 4160, 64)]:
        Kr = -(-K // g) * g
        w = w16_word_index(M, Kr)   # the decoder the GPU parity tests read the kernel's rows with
        assert len(np.unique(w)) == w.size, (M, K, g)
        assert w.max() * 16 + 16 <= B.convrot_w4a16_workspace_bytes(M, K, g), (M, K, g)


def test_w4a16_sizes_and_statuses():
    # rows rounded up to 16 and K to 128, bf16 each
    assert B.convrot_w4a16_workspace_bytes(1, 3072, 256) == 16 * 3072 * 2
    assert B.convrot_w4a16_workspace_bytes(32, 12288, 256) == 32 * 12288 * 2
    assert B.convrot_w4a16_workspace_bytes(3, 192, 64) == 16 * 256 * 2
    assert B.convrot_w4a16_workspace_bytes(17, 1000, 256) == 32 * 1024 * 2   # K_rot = 1024
    assert B.convrot_w4a16_workspace_bytes(0, 1024, 256) == 0
    with pytest.raises(B.ConvRotError):
        B.convrot_w4a16_workspace_bytes(33, 1024, 256)                    # M > 32: the W4A4 path's regime
    ok = B.convrot_w4a16_workspace_bytes(16, 1024, 256)

    def v(**over):
        args = dict(X=4096, M=16, K=1024, image=8192, sw=16384, bias=0, N=1024, g=256, Y=32768, ws=65536,
                    ws_bytes=ok)
        args.update(over)
        return B.convrot_validate_linear_w4a16(*[args[k] for k in ("X", "M", "K", "image", "sw", "bias", "N", "g",
                                                                     "Y", "ws", "ws_bytes")])

    assert v() == B.CONVROT_OK
    assert v(M=33) == B.CONVROT_EINVAL
    assert v(g=256 | B.CONVROT_REGULAR_HADAMARD) == B.CONVROT_OK
    assert v(ws_bytes=ok - 1) == B.CONVROT_EWORKSPACE
    assert v(X=4100) == B.CONVROT_EINVAL
    assert v(M=0, X=0, Y=0) == B.CONVROT_OK


def test_validate_weight_statuses():
    assert B.convrot_validate_weight(4096, 1024, 1024, 256, 8192, 16384) == B.CONVROT_OK
    assert B.convrot_validate_weight(4096, 1024, 1024, 32, 8192, 16384) == B.CONVROT_EINVAL
    assert B.convrot_validate_weight(0, 1024, 1024, 256, 8192, 16384) == B.CONVROT_EINVAL
    assert B.convrot_validate_weight(4096, 1024, 1000, 64, 8192, 16384) == B.CONVROT_OK     # padded to 1024
    assert B.convrot_validate_weight(4096, 1024, 1001, 64, 8192, 16384) == B.CONVROT_EINVAL  # K % 8 != 0
    assert B.convrot_validate_weight(0, 0, 1024, 256, 0, 0) == B.CONVROT_OK


def test_binding_size_limits_match_the_library():
    v = B.convrot_validate_weight
    assert v(4096, 1, B.MAX_K, 256, 8192, 16384) == B.CONVROT_OK
    assert v(4096, 1, B.MAX_K + 8, 256, 8192, 16384) == B.CONVROT_EINVAL
    assert v(4096, 1, B.MAX_K - 8, 256, 8192, 16384) == B.CONVROT_OK       # rotated width MAX_K
    assert v(4096, B.MAX_ROWS, 1024, 256, 8192, 16384) == B.CONVROT_OK
    assert v(4096, B.MAX_ROWS + 1, 1024, 256, 8192, 16384) == B.CONVROT_EINVAL


# --------------------------------------------------------------------------
# host layout tools vs the oracle
# --------------------------------------------------------------------------

@pytest.mark.parametrize("N,K", [(32, 128), (48, 256), (70, 192), (1, 64)])
def test_host_pack_and_transpose_match_oracle(N, K):
    rng = np.random.default_rng(N * 1000 + K)
    codes = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    nk = B.convrot_host_pack_nk(codes)
    assert np.array_equal(nk, oracle.pack_nk(codes))
    assert np.array_equal(B.convrot_host_unpack_nk(nk, K), codes)
    if N % 2 == 0:
        kn = B.convrot_host_nk_to_kn(nk, N, K)
        assert np.array_equal(kn, oracle.nk_to_kn(nk, N, K))
        assert np.array_equal(B.convrot_host_kn_to_nk(kn, N, K), nk)


@pytest.mark.parametrize("N,K", [(32, 128), (64, 384), (70, 192), (5, 64), (96, 1024)])
def test_host_image_round_trip(N, K):
    rng = np.random.default_rng(7 + N + K)
    codes = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    nk = oracle.pack_nk(codes)
    image = B.convrot_host_nk_to_image(nk, N, K)
    assert image.size == B.convrot_weight_image_bytes(N, K, 64)
    assert np.array_equal(B.convrot_host_image_to_nk(image, N, K), nk)
    assert np.array_equal(B.convrot_host_image_fp6_to_nk(image, N, K), nk)
    # every code lands somewhere and the padding is zero: the INT4 part holds
    # exactly the nibbles of nk (as a multiset) plus zeros
    int4 = image[:_int4_plane(N, K)]
    nz_img = np.count_nonzero(np.concatenate([int4 & 0xF, int4 >> 4]))
    nz_nk = np.count_nonzero(np.concatenate([nk & 0xF, nk >> 4]))
    assert nz_img == nz_nk


def test_host_image_widening_property():
    """Inside the image, (word << 4) & 0xF0F0F0F0 and word & 0xF0F0F0F0 are
    16 x the codes k..k+3 and k+4..k+7 as signed bytes (checked on a unit)."""
    N, K = 32, 128
    rng = np.random.default_rng(1)
    codes = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    image = B.convrot_host_nk_to_image(oracle.pack_nk(codes), N, K)
    words = image[:_int4_plane(N, K)].view(np.uint32)
    lo = ((words << 4) & 0xF0F0F0F0).astype(np.uint32).view(np.int8).astype(np.int32)
    hi = (words & 0xF0F0F0F0).astype(np.uint32).view(np.int8).astype(np.int32)
    assert np.all(lo % 16 == 0) and np.all(hi % 16 == 0)
    got = np.sort(np.concatenate([lo, hi]) // 16)
    assert np.array_equal(got, np.sort(codes.ravel().astype(np.int32)))


def _e2m3_value(v):
    """OCP MX FP6 E2M3: sign bit 5, exponent bits 4..3 (bias 1), mantissa bits
    2..0; exponent 0 is subnormal (m / 8)."""
    sign = -1.0 if v & 0x20 else 1.0
    e, m = (v >> 3) & 3, v & 7
    return sign * (m / 8.0 if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 8.0))


@pytest.mark.parametrize("N,K", [(32, 128), (70, 192), (5, 64)])
def test_host_image_fp6_plane_by_definition(N, K):
    """The FP6 part of a weight image, decoded here from its documented layout
    (32-row x 128-K units of 3072 bytes; row r at 96 r; four 24-byte blocks per
    row, block b holding codes 32 b + e at bit 6 e, stored at block position
    b ^ f(r), f(r) = 2 r3 + (r2 xor r4) from the bits of r) with the OCP e2m3
    value rule, gives back every code; padding decodes to 0."""
    rng = np.random.default_rng(N + 3 * K)
    codes = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    image = B.convrot_host_nk_to_image(oracle.pack_nk(codes), N, K)
    plane = image[_int4_plane(N, K):]
    Np, Kp = -(-N // 32) * 32, -(-K // 128) * 128
    assert plane.size == Np * Kp * 3 // 4
    KB = Kp // 128
    got = np.zeros((Np, Kp))
    for n in range(Np):
        for kb in range(KB):
            base = ((n // 32) * KB + kb) * 3072 + (n % 32) * 96
            phys = plane[base:base + 96]
            logical = np.empty(96, np.uint8)
            r = n % 32
            f = (((r >> 3) & 1) << 1) | (((r >> 2) ^ (r >> 4)) & 1)
            for blk in range(4):
                src = blk ^ f
                logical[24 * blk:24 * blk + 24] = phys[24 * src:24 * src + 24]
            bits = np.unpackbits(logical, bitorder="little")
            for kl in range(128):
                v = int(sum(int(bits[6 * kl + i]) << i for i in range(6)))
                got[n, kb * 128 + kl] = _e2m3_value(v)
    assert np.array_equal(got[:N, :K], codes.astype(np.float64))
    assert np.all(got[N:] == 0) and np.all(got[:, K:] == 0)
