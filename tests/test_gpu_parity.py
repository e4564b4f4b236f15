"""Parity of the HIP path (through the C ABI) with the CPU oracle, on seeded
synthetic inputs.  Small shapes span several tiles with ragged tails; the
full diffusion-transformer shapes run in the launch configuration the
benchmark times.  Every output is compared element by element.

Method: convrot-mlx README, "What is included" (grouped normalized Hadamard
rotation for g = 64/256, symmetric rowwise absmax INT4 in [-7, 7],
reversible packed layouts), "Install and test" (rotation, activation
quantization, integer product, scaling, bias); comfy-quants issue "convrot
is ... QuaRot Stage 1c", section 1 (R = I_G (x) H)."""
import numpy as np
import pytest

import oracle
from w4a4_rotated_bit_amd import synth

from w4a4_rotated_bit_amd.binding import CONVROT_TILE_FP6
from ._parity import compare_codes, compare_rotated, compare_y, w16_word_index

pytestmark = pytest.mark.gpu


def _dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def _w16_rows(ws, M, Kr):
    """The bf16 rotated rows [M][Kr] out of a W4A16 workspace, decoded by the
    layout that include/convrot.h states for it (16-byte words in the order
    of 16-row blocks, 128-K units, steps j, quarters q, rows)."""
    words = ws.cpu().numpy().view(np.uint16).reshape(-1, 8)
    return words[w16_word_index(M, Kr)].reshape(M, Kr)


def _host_bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


# --------------------------------------------------------------------------
# rotation + quantization (K1)
# --------------------------------------------------------------------------

PREP_SHAPES = [
    (5, 256, 256), (37, 1024, 256), (64, 3072, 256), (3, 12288, 256), (2, 16384, 256),
    (7, 192, 64), (128, 2048, 64), (1, 64, 64), (33, 1024, 64),
]


REG = 0x10000  # the library's regular-Hadamard flag (checked against the header in test_abi)
INT4 = 0x20000  # the library's INT4-only image flag (checked against the header in test_abi)
PREP_SHAPES += [(5, 256, 256 | REG), (37, 3072, 256 | REG), (2, 16384, 256 | REG), (7, 192, 64 | REG),
                (33, 1024, 64 | REG), (1, 64, 64 | REG),
                # K not a multiple of g (zero-padded last group), both matrices
                (6, 328, 256), (3, 3000, 256), (9, 200, 64), (2, 8, 64), (4, 776, 256 | REG), (5, 1000, 64 | REG)]


@pytest.mark.parametrize("rows,K,g", PREP_SHAPES)
def test_prepare_rows_parity(gpu, rows, K, g):
    x = synth.random_bf16((rows, K), seed=rows * 7 + K + g, outliers=max(1, K // 200))
    x[0, :] = 0  # an all-zero row
    q, s, r = gpu.convrot_prepare_rows(_dev(x), g, want_rotated=True)
    oq, os_, orr = oracle.prepare_rows(x, g, want_rotated=True)
    gq, gs, gr = q.cpu().numpy(), s.cpu().numpy(), r.cpu().numpy()
    compare_rotated(gr, orr)
    assert np.array_equal(gs, os_), "scales differ"
    compare_codes(gq, oq, orr, os_)
    assert gs[0] == 0 and np.all(gq[0] == 0)


def test_prepare_rows_golden_ties(gpu):
    import json
    import os
    from fractions import Fraction
    with open(os.path.join(os.path.dirname(__file__), "golden", "quant_ties.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        g, K = case["g"], case["K"]
        x = np.zeros((K,), dtype=np.float32)
        for gi, grp in enumerate(case["groups"]):
            x[gi * g:(gi + 1) * g:2] = float(Fraction(grp["x_even"]))
            x[gi * g + 1:(gi + 1) * g:2] = float(Fraction(grp["x_odd"]))
        q, s, _ = gpu.convrot_prepare_rows(_dev(synth.to_bf16_bits(x)[None, :]), g)
        want = np.zeros((K,), np.int8)
        for k, v in case["codes_nonzero"].items():
            want[int(k)] = v
        assert np.array_equal(q.cpu().numpy()[0], want), case["name"]
        assert float(s.cpu().numpy()[0]) == float(Fraction(case["scale"])), case["name"]


# --------------------------------------------------------------------------
# weight preparation and layouts (K1 + K3)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("N,K,g", [(70, 512, 256), (32, 256, 256), (45, 192, 64), (256, 1024, 64),
                                   # K not a multiple of g: the last group is zero-padded
                                   (33, 328, 256), (40, 200, 64)])
def test_weight_image_and_nk_parity(gpu, N, K, g):
    w = synth.random_bf16((N, K), seed=N + K, std=0.02)
    K = gpu.rotated_width(K, g)   # code width
    oq, osw = oracle.prepare_weight(w, g)
    onk = oracle.pack_nk(oq)
    W = _dev(w)
    image, sw = gpu.convrot_prepare_weight(W, g)
    nk, sw2 = gpu.convrot_quantize_weight(W, g)
    osr = oracle.rotate_rows(w, g)
    assert np.array_equal(sw.cpu().numpy(), osw) and np.array_equal(sw2.cpu().numpy(), osw)
    img = image.cpu().numpy()
    compare_codes(oracle.unpack_nk(gpu.convrot_host_image_to_nk(img, N, K), K), oq, osr, osw, "image codes")
    compare_codes(oracle.unpack_nk(nk.cpu().numpy(), K), oq, osr, osw, "nk codes")
    # the FP6 copy in the image holds the same codes
    assert np.array_equal(gpu.convrot_host_image_fp6_to_nk(img, N, K), gpu.convrot_host_image_to_nk(img, N, K))
    # the device repack of N x packed-K is byte-identical to the direct image
    image2 = gpu.convrot_repack_nk_to_image(nk, N, K, g)
    assert np.array_equal(image2.cpu().numpy(), img)
    # and so is the host repack (layout definition shared by host and device)
    assert np.array_equal(gpu.convrot_host_nk_to_image(nk.cpu().numpy(), N, K), img)
    # lossless round trip through K x packed-N
    if N % 2 == 0:
        kn = gpu.convrot_host_nk_to_kn(nk.cpu().numpy(), N, K)
        assert np.array_equal(kn, oracle.nk_to_kn(onk, N, K))
        assert np.array_equal(gpu.convrot_host_kn_to_nk(kn, N, K), onk)


# --------------------------------------------------------------------------
# integer product (K2 without the epilogue)
# --------------------------------------------------------------------------

GEMM_SHAPES = [(1, 32, 128), (37, 70, 384), (256, 256, 1024), (300, 520, 1152), (64, 1024, 3072),
               (513, 257, 256), (17, 33, 12288), (5, 100, 2560), (32, 64, 640), (3, 4000, 3072),
               (256, 512, 8192), (100, 300, 6144), (20, 9000, 1024), (7, 17000, 256),
               # FP6 256 x 256 block tiles (216 and 192 of them, also ragged), FP6 192 x 384
               # (256 of them, also ragged), INT8 192 x 192 split 2 ways along K, and
               # 192 x 192 split 8 ways (256 workgroups, also ragged): the shapes the plan
               # picks here (convrot_linear_plan)
               (1536, 9216, 128), (1500, 9000, 256), (1536, 12288, 128), (1500, 12000, 384),
               (1536, 3072, 8192), (4096, 3072, 128), (4000, 3000, 256), (256, 3072, 16384),
               (200, 3011, 16384),
               # the two FP6 tiles with at least eight 128-K blocks, so that their K loops
               # run the steady state of the stage ring (aligned and ragged)
               (1536, 9216, 1024), (1500, 9000, 1152), (1536, 12288, 1024), (1500, 12000, 1408),
               # the weight stream with 2, 3 and 4 groups of 32 rows (M <= 128; strips padded
               # to a multiple of 8), and the first M past it (block tiles)
               (33, 130, 384), (64, 1000, 1152), (65, 512, 2048), (128, 2048, 2048), (127, 33, 640),
               (129, 200, 1024)]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_i32_bit_exact(gpu, M, N, K):
    rng = np.random.default_rng(M * 31 + N * 7 + K)
    qx = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    qw = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    image = _dev(gpu.convrot_host_nk_to_image(oracle.pack_nk(qw), N, K))
    acc = gpu.convrot_gemm_i32(_dev(qx), image, N).cpu().numpy()
    assert np.array_equal(acc, oracle.gemm_i32(qx, qw))


def test_gemm_i32_integer_edges(gpu):
    K = 12288
    qx = np.stack([np.full(K, 7, np.int8), np.full(K, -7, np.int8), np.zeros(K, np.int8)])
    qw = np.stack([np.full(K, 7, np.int8), np.full(K, -7, np.int8)] * 16)
    image = _dev(gpu.convrot_host_nk_to_image(oracle.pack_nk(qw), 32, K))
    acc = gpu.convrot_gemm_i32(_dev(qx), image, 32).cpu().numpy()
    assert acc[0, 0] == 49 * K and acc[0, 1] == -49 * K and acc[1, 0] == -49 * K and acc[1, 1] == 49 * K
    assert np.all(acc[2] == 0)
    assert np.array_equal(acc, oracle.gemm_i32(qx, qw))


# (tile, splits, M, N, K): every block tile at shapes the plan would not give
# it, unsplit and (192 x 192) split
F6 = CONVROT_TILE_FP6  # or-ed into tile_n: the FP6 tile of size 192 x 384
TILED = [((256, 256), 1, 300, 520, 1152), ((256, 256), 1, 33, 1000, 2048), ((256, 256), 1, 700, 300, 5120),
         # the FP6 192 x 384 tile and its two-stage ring: 1, 2, 3 and many K blocks, ragged
         ((192, 384 | F6), 1, 300, 700, 128), ((192, 384 | F6), 1, 200, 500, 256), ((192, 384 | F6), 1, 40, 3000, 384),
         ((192, 384 | F6), 1, 1000, 400, 6144), ((192, 384 | F6), 1, 385, 769, 1152),
         ((192, 384), 1, 300, 700, 2048), ((192, 384), 1, 1000, 400, 6144), ((192, 384), 1, 40, 3000, 1024),
         ((192, 192), 1, 1536, 9216, 1024), ((192, 192), 3, 256, 600, 6144), ((192, 192), 8, 200, 3011, 16384),
         ((192, 192), 5, 500, 260, 8192)]


@pytest.mark.parametrize("tile,splits,M,N,K", TILED)
def test_gemm_i32_every_block_tile(gpu, tile, splits, M, N, K):
    rng = np.random.default_rng(M + 3 * N + 5 * K + splits)
    qx = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    qw = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    image = _dev(gpu.convrot_host_nk_to_image(oracle.pack_nk(qw), N, K))
    acc, ws = gpu.convrot_gemm_i32_tiled(_dev(qx), image, N, tile, splits)
    assert np.array_equal(acc.cpu().numpy(), oracle.gemm_i32(qx, qw))
    assert gpu.workspace_status(ws) == 0


@pytest.mark.parametrize("tile,splits", [((256, 256), 1), ((192, 384), 1), ((192, 192), 8), ((192, 192), 1),
                                         ((192, 384 | F6), 1)])
def test_gemm_i32_saturated_codes_on_every_block_tile(gpu, tile, splits):
    """Integer edges at the longest rows: every code +-7 and K = 16384, so that
    |acc| reaches 49 K = 802,816 -- through each block tile (on the FP6 tile the
    binary32 sums stay exact integers below 2^24)."""
    K, M, N = 16384, 64, 96
    rng = np.random.default_rng(7)
    sx = rng.choice(np.array([-1, 1], np.int8), size=(M, K))
    sw = rng.choice(np.array([-1, 1], np.int8), size=(N, K))
    sx[0], sx[1], sw[0], sw[1] = 1, -1, 1, -1
    sw[2] = sx[5]
    qx, qw = (7 * sx).astype(np.int8), (7 * sw).astype(np.int8)
    image = _dev(gpu.convrot_host_nk_to_image(oracle.pack_nk(qw), N, K))
    acc = gpu.convrot_gemm_i32_tiled(_dev(qx), image, N, tile, splits)[0].cpu().numpy()
    assert acc[0, 0] == 49 * K and acc[0, 1] == -49 * K and acc[1, 0] == -49 * K and acc[1, 1] == 49 * K
    assert acc[5, 2] == 49 * K
    assert np.array_equal(acc, oracle.gemm_i32(qx, qw))


@pytest.mark.parametrize("tile,splits,M,N,K", [((256, 256), 2, 300, 520, 4096), ((192, 384), 2, 300, 700, 4096),
                                               ((256, 256), 3, 1536, 3072, 12288), ((192, 384), 4, 1536, 3072, 12288),
                                               ((192, 384 | F6), 2, 300, 700, 4096),
                                               ((192, 384 | F6), 3, 1536, 3072, 12288)])
def test_gemm_i32_split_k_on_the_eight_wave_tiles(gpu, tile, splits, M, N, K):
    """The split-K exchange on the eight-wave block tiles, which the plan
    itself never splits, including the down-projection shape with the splits
    a timing probe once forced there when the GPU faulted.  Such a split needs
    more partial-tile room than a workspace sized by the library's own plan
    (checked on the CPU in test_abi); here the workspace is sized from the
    forced plan, as the hook requires."""
    rng = np.random.default_rng(M + N + K + splits)
    qx = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    qw = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    image = _dev(gpu.convrot_host_nk_to_image(oracle.pack_nk(qw), N, K))
    assert gpu.convrot_split_k_extent(M, K, N, tile, splits)["partial_end"] > 0
    acc, ws = gpu.convrot_gemm_i32_tiled(_dev(qx), image, N, tile, splits)
    assert np.array_equal(acc.cpu().numpy(), oracle.gemm_i32(qx, qw))
    assert gpu.workspace_status(ws) == 0


def test_split_k_timeout_is_reported(gpu):
    """The split-K finalizer's bounded wait, forced to run out from the host
    (it waits for one writer more than exist, with a tiny bound): the kernel
    still ends, the workspace's status word says so, and the next call on the
    same workspace (whose activation step clears the counters and the status)
    is exact again."""
    import torch
    M, N, K = 256, 600, 6144
    rng = np.random.default_rng(11)
    qx = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    qw = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    image = _dev(gpu.convrot_host_nk_to_image(oracle.pack_nk(qw), N, K))
    _, ws = gpu.convrot_gemm_i32_tiled(_dev(qx), image, N, (192, 192), 3, test_flags=gpu.CONVROT_TEST_SPLIT_TIMEOUT)
    torch.cuda.synchronize()
    assert gpu.workspace_status(ws) == gpu.CONVROT_STATUS_SPLIT_TIMEOUT
    acc, ws = gpu.convrot_gemm_i32_tiled(_dev(qx), image, N, (192, 192), 3, workspace=ws)
    torch.cuda.synchronize()
    assert gpu.workspace_status(ws) == 0
    assert np.array_equal(acc.cpu().numpy(), oracle.gemm_i32(qx, qw))


@pytest.mark.parametrize("M,N,K", [(256, 256, 4096), (160, 1024, 8192), (300, 700, 4096), (256, 4096, 12288)])
def test_split_k_workspace_reuse(gpu, M, N, K):
    """Shapes whose tiles are split along K: a workspace full of garbage is
    cleared by the activation step, and repeated GEMMs on one workspace (the
    split-K counters are returned to zero by each launch) -- also with a
    different N in between -- give identical, oracle-exact results."""
    import torch
    # the workspace holds split-K partial tiles only when the GEMM splits K
    assert gpu.convrot_workspace_bytes(M, K, N, 256) > gpu.convrot_workspace_bytes(M, K, 0, 256)
    x = synth.random_bf16((M, K), seed=M + K, outliers=4)
    w = synth.random_bf16((N, K), seed=N + K + 1, std=0.02)
    b = synth.random_bf16((N,), seed=N, std=0.01)
    oq_w, osw = oracle.prepare_weight(w, 256)
    y_or = oracle.linear(x, oq_w, osw, b, 256)
    image, sw = gpu.convrot_prepare_weight(_dev(w), 256)
    ws = gpu.new_workspace(M, K, N, 256)
    ws.fill_(0xFF)
    gpu.convrot_prepare_activations(_dev(x), 256, ws)
    # not knowing N, the activation step writes both copies of the codes
    torch.cuda.synchronize()
    assert np.array_equal(gpu.convrot_host_workspace_fp6_codes(ws, M, K), gpu.workspace_act_codes(ws, M, K))
    outs = [gpu.convrot_gemm(ws, M, K, image, sw, _dev(b), N, 256) for _ in range(3)]
    # a narrower GEMM on the same workspace, then the original again
    Nn = N // 2
    gpu.convrot_gemm(ws, M, K, image, sw, _dev(b), Nn, 256)
    outs.append(gpu.convrot_gemm(ws, M, K, image, sw, _dev(b), N, 256))
    torch.cuda.synchronize()
    for Y in outs:
        assert np.array_equal(_host_bits(Y), y_or)


# --------------------------------------------------------------------------
# the whole linear
# --------------------------------------------------------------------------

def _linear_act_codes(gpu, ws, M, K, N, g):
    """The activation codes convrot_linear leaves in its workspace, from the copy
    its plan reads (FP6 for the FP6 block tile, else the INT4 image)."""
    if M > 32 and gpu.convrot_linear_plan(M, K, N, g)["mfma"] == gpu.CONVROT_MFMA_FP6:
        return gpu.convrot_host_workspace_fp6_codes(ws, M, gpu.rotated_width(K, g))
    return gpu.workspace_act_codes(ws, M, gpu.rotated_width(K, g))


def _oracle_g(g):
    """The group argument for the oracle: the INT4-only image flag is a storage
    choice of the library and has no arithmetic meaning."""
    return g & ~INT4


def _linear_parity(gpu, x, w, bias, g):
    N, K = w.shape
    og = _oracle_g(g)
    oq_w, osw = oracle.prepare_weight(w, og)
    y_or, parts = oracle.linear(x, oq_w, osw, bias, og, want_parts=True)
    image, sw = gpu.convrot_prepare_weight(_dev(w), g)
    ws = gpu.new_workspace(x.shape[0], K, N, g)
    Y = gpu.convrot_linear(_dev(x), image, sw, None if bias is None else _dev(bias), N, g, workspace=ws)
    gy = _host_bits(Y)
    # codes of X (from the copy of the workspace the plan reads) and of W (from
    # the image), K_rot wide
    M = x.shape[0]
    qx = _linear_act_codes(gpu, ws, M, K, N, g)
    K = gpu.rotated_width(K, g)
    orx = oracle.rotate_rows(x, og)
    compare_codes(qx, parts["qx"], orx, parts["sx"], "activation codes")
    qw = oracle.unpack_nk(gpu.convrot_host_image_to_nk(image.cpu().numpy(), N, K), K)
    compare_codes(qw, oq_w, oracle.rotate_rows(w, og), osw, "weight codes")
    rows_ok = np.all(qx == parts["qx"], axis=1) & bool(np.array_equal(qw, oq_w))
    compare_y(gy, y_or, rows_ok)
    return gy, y_or


@pytest.mark.parametrize("name", ["tiny_m64_k1024_n1024_g256", "g64_m128_k2048_n2048"])
def test_linear_small_workloads_full(gpu, name):
    inp = synth.make(name)
    wl = inp["workload"]
    _linear_parity(gpu, inp["x"], inp["w"], inp["bias"], wl.g)


@pytest.mark.parametrize("M,N,K,g", [(1, 96, 256, 256), (37, 70, 512, 256), (300, 520, 1280, 256),
                                     (33, 64, 192, 64), (257, 300, 2048, 64), (2, 2, 64, 64),
                                     # M <= 4: the single-kernel path (1..3 strips per workgroup, 1..4 waves per row)
                                     (1, 100, 1024, 256), (3, 5000, 4096, 256), (4, 33, 512, 64),
                                     (2, 17000, 2048, 64), (4, 48, 1280, 256), (1, 12288, 3072, 256),
                                     # the regular Hadamard matrix, both paths
                                     (37, 70, 512, 256 | REG), (257, 300, 2048, 64 | REG),
                                     (1, 100, 1024, 256 | REG), (4, 33, 512, 64 | REG),
                                     (3, 5000, 4096, 256 | REG),
                                     # K not a multiple of g, both paths
                                     (37, 70, 328, 256), (300, 520, 1000, 64), (1, 100, 1000, 256),
                                     (4, 33, 2000, 64 | REG), (65, 200, 3000, 256 | REG)])
def test_linear_ragged_shapes(gpu, M, N, K, g):
    x = synth.random_bf16((M, K), seed=M + N, outliers=3)
    w = synth.random_bf16((N, K), seed=N + K, std=0.02)
    b = synth.random_bf16((N,), seed=K, std=0.01)
    _linear_parity(gpu, x, w, b, g)


@pytest.mark.parametrize("M,N,K,g,bias", [
    # the FP6 256 x 256 and 192 x 384 tiles through the whole linear, ragged M and N
    # (N % 8 != 0: the epilogue's partial 16-byte stores), with and without bias
    (1500, 9000, 3072, 256, True), (1501, 9004, 3072, 256, False), (1500, 12000, 3072, 256, True),
    (1499, 12004, 3072, 256, False), (300, 700, 1152, 256, False),
    # INT4-only weight images: every product on the INT8 matrix cores, including the
    # shapes the FP6 tile takes otherwise, the weight-streaming and one-kernel paths
    (1500, 9000, 3072, 256 | INT4, True), (300, 520, 1280, 256 | INT4, False), (40, 1000, 2048, 64 | INT4, True),
    (16, 3000, 3072, 256 | INT4, True), (3, 5000, 4096, 256 | INT4 | REG, True), (65, 200, 3000, 256 | INT4, True)])
def test_linear_block_tiles_and_image_formats(gpu, M, N, K, g, bias):
    x = synth.random_bf16((M, K), seed=M + 2 * N, outliers=3)
    w = synth.random_bf16((N, K), seed=N + 3 * K, std=0.02)
    b = synth.random_bf16((N,), seed=K + 1, std=0.01) if bias else None
    _linear_parity(gpu, x, w, b, g)


def test_int4_image_is_the_int4_part_of_the_full_image(gpu):
    """An INT4-only image is byte for byte the first part of the default image
    (0.5 bytes per weight, padding included), and the linear on it gives the
    same Y as the FP6 tile on the full image (both are exact integer products)."""
    M, N, K = 1536, 9216, 1024
    x = synth.random_bf16((M, K), seed=91, outliers=4)
    w = synth.random_bf16((N, K), seed=92, std=0.02)
    b = synth.random_bf16((N,), seed=93, std=0.01)
    full, sw = gpu.convrot_prepare_weight(_dev(w), 256)
    int4, sw4 = gpu.convrot_prepare_weight(_dev(w), 256 | INT4)
    assert int4.numel() == N * K // 2 == gpu.convrot_weight_image_bytes(N, K, 256 | INT4)
    assert np.array_equal(int4.cpu().numpy(), full.cpu().numpy()[:int4.numel()])
    assert gpu.convrot_linear_plan(M, K, N, 256)["mfma"] == gpu.CONVROT_MFMA_FP6
    assert gpu.convrot_linear_plan(M, K, N, 256 | INT4)["mfma"] == gpu.CONVROT_MFMA_I8
    y6 = _host_bits(gpu.convrot_linear(_dev(x), full, sw, _dev(b), N, 256))
    y4 = _host_bits(gpu.convrot_linear(_dev(x), int4, sw4, _dev(b), N, 256 | INT4))
    assert np.array_equal(y6, y4)


def test_linear_no_bias_and_zero_rows(gpu):
    M, N, K, g = 40, 64, 512, 256
    x = synth.random_bf16((M, K), seed=3, outliers=2)
    x[5] = 0
    x[39] = 0
    w = synth.random_bf16((N, K), seed=4, std=0.02)
    gy, _ = _linear_parity(gpu, x, w, None, g)
    assert np.all(gy[5] == 0) and np.all(gy[39] == 0)
    b = synth.random_bf16((N,), seed=5, std=0.01)
    gy, _ = _linear_parity(gpu, x, w, b, g)
    assert np.array_equal(gy[5], b) and np.array_equal(gy[39], b)


def test_linear_empty_is_noop(gpu):
    import torch
    w = synth.random_bf16((32, 256), seed=1, std=0.02)
    image, sw = gpu.convrot_prepare_weight(_dev(w), 256)
    X = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    Y = gpu.convrot_linear(X, image, sw, None, 32, 256, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    assert Y.shape == (0, 32)


def test_linear_rejects_bad_arguments(gpu):
    import torch
    w = synth.random_bf16((32, 256), seed=1, std=0.02)
    image, sw = gpu.convrot_prepare_weight(_dev(w), 256)
    X = _dev(synth.random_bf16((4, 256), seed=2))
    with pytest.raises(gpu.ConvRotError) as e:
        gpu.convrot_linear(X, image, sw, None, 32, 128)
    assert e.value.status == gpu.CONVROT_EINVAL
    with pytest.raises(gpu.ConvRotError) as e:
        gpu.convrot_linear(X, image, sw, None, 32, 256, workspace=torch.empty(64, dtype=torch.uint8, device="cuda"))
    assert e.value.status == gpu.CONVROT_EWORKSPACE


# --------------------------------------------------------------------------
# W4A16 variant (M <= 32)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K,g", [(1, 96, 256, 256), (4, 5000, 3072, 256), (16, 12288, 3072, 256),
                                     (17, 300, 1024, 64), (32, 1000, 2048, 256 | REG), (5, 70, 192, 64),
                                     (3, 17000, 512, 64 | REG), (1, 12288, 3072, 256), (2, 300, 1000, 256)])
def test_linear_w4a16(gpu, M, N, K, g):
    """The bf16 rotated rows are bit-exact (one rounding of the exact
    rotation); Y is within the path's tolerance of the oracle, whose sum is
    exact where the matrix cores accumulate in binary32."""
    import torch
    x = synth.random_bf16((M, K), seed=M * 3 + K, outliers=3)
    w = synth.random_bf16((N, K), seed=N + 5, std=0.02)
    b = synth.random_bf16((N,), seed=N + 6, std=0.01)
    oq_w, osw = oracle.prepare_weight(w, g)
    y_or, xr_or = oracle.linear_w4a16(x, oq_w, osw, b, g, want_rotated=True)
    image, sw = gpu.convrot_prepare_weight(_dev(w), g)
    ws = torch.zeros(gpu.convrot_w4a16_workspace_bytes(M, K, g), dtype=torch.uint8, device="cuda")
    Y = gpu.convrot_linear_w4a16(_dev(x), image, sw, _dev(b), N, g, workspace=ws)
    torch.cuda.synchronize()
    Kr = gpu.rotated_width(K, g)
    assert ws.numel() == -(-M // 16) * 16 * -(-Kr // 128) * 128 * 2
    assert np.array_equal(_w16_rows(ws, M, Kr), xr_or), "bf16 rotated rows differ"
    gy = synth.bf16_bits_to_f32(_host_bits(Y)).astype(np.float64)
    oy = synth.bf16_bits_to_f32(y_or).astype(np.float64)
    err = np.abs(gy - oy).max() / np.abs(oy).max()
    assert err <= 1e-2, f"max |dY| / max |Y| = {err:.3g}"
    assert np.mean(gy == oy) > 0.5          # most values round to the same bf16


@pytest.mark.parametrize("K,N,g", [(3072, 12288, 256), (1000, 700, 256), (512, 300, 64 | REG), (2048, 129, 64)])
def test_single_kernel_paths_match_two_kernel_paths(gpu, K, N, g):
    """Rows are independent, so the first four rows of a five-row input (two
    launches: prep, then the weight-streaming product) and the same four rows
    alone (one launch that rotates the rows in every workgroup) must agree bit
    for bit -- for W4A4 and for W4A16, whose binary32 sums are taken in the
    same order on both paths."""
    x = synth.random_bf16((5, K), seed=K + N, outliers=2)
    w = synth.random_bf16((N, K), seed=N + 1, std=0.02)
    b = synth.random_bf16((N,), seed=N + 2, std=0.01)
    image, sw = gpu.convrot_prepare_weight(_dev(w), g)
    Kr = gpu.rotated_width(K, g)
    assert gpu.convrot_linear_kernel_count(4, K, N, g) == 1 and gpu.convrot_linear_kernel_count(5, K, N, g) == 2
    for fn in (gpu.convrot_linear, gpu.convrot_linear_w4a16):
        y5 = _host_bits(fn(_dev(x), image, sw, _dev(b), N, g))
        y4 = _host_bits(fn(_dev(x[:4]), image, sw, _dev(b), N, g))
        assert np.array_equal(y4, y5[:4]), fn.__name__
    # the one-launch W4A16 path leaves the bf16 rows in the workspace as the two-launch path does
    import torch
    ws4 = torch.zeros(gpu.convrot_w4a16_workspace_bytes(4, K, g), dtype=torch.uint8, device="cuda")
    ws5 = torch.zeros(gpu.convrot_w4a16_workspace_bytes(5, K, g), dtype=torch.uint8, device="cuda")
    gpu.convrot_linear_w4a16(_dev(x[:4]), image, sw, _dev(b), N, g, workspace=ws4)
    gpu.convrot_linear_w4a16(_dev(x), image, sw, _dev(b), N, g, workspace=ws5)
    torch.cuda.synchronize()
    assert np.array_equal(_w16_rows(ws4, 4, Kr), _w16_rows(ws5, 5, Kr)[:4])


@pytest.mark.parametrize("kind", [1, 2])
def test_matrix_core_probe_runs(gpu, kind):
    """The measurement hook: the MFMA count it reports follows its launch
    shape (two four-wave workgroups per CU), and it ends normally."""
    import torch
    count, out = gpu.convrot_matrix_core_probe(kind, 8)
    torch.cuda.synchronize()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert count == 2 * cus * 4 * 8 * 4
    assert out.numel() == 2 * cus * 256
    with pytest.raises(gpu.ConvRotError):
        gpu.convrot_matrix_core_probe(kind, 8, out=out[:16])


FULL = ["flux_qkv_m1536_k3072_n9216", "flux_mlp_up_m1536_k3072_n12288", "flux_mlp_down_m1536_k12288_n3072",
        "decode_m1_k3072_n12288", "decode_m4_k3072_n12288", "decode_m16_k3072_n12288", "stress_m4096_k3072_n3072"]


@pytest.mark.parametrize("name", FULL + ["flux_qkv_m1536_k3072_n9216+regular", "flux_qkv_m1536_k3072_n9216+zero_rows",
                                         "decode_m4_k3072_n12288+zero_rows", "flux_qkv_m1536_k3072_n9216+int4",
                                         "flux_mlp_down_m1536_k12288_n3072+regular",
                                         # the FP6 192 x 384 tile behind the other prep instances, and
                                         # the INT8 192 x 384 tile (with the streamed X reads) at full size
                                         "flux_mlp_up_m1536_k3072_n12288+regular", "flux_mlp_up_m1536_k3072_n12288+g64",
                                         "flux_mlp_up_m1536_k3072_n12288+int4",
                                         # 4096 rows on INT8 192 x 384 tiles: a ragged last row of tiles
                                         "stress_m4096_k3072_n3072+int4",
                                         # the weight stream behind the group-64 prep
                                         "decode_m16_k3072_n12288+g64"])
def test_linear_full_size(gpu, name):
    """Full shapes, in the launch configuration the benchmark times, against
    the oracle on every output: all activation and weight codes, the scales,
    and Y element by element.  "+regular": the same inputs rotated with the
    regular Hadamard matrix.  "+zero_rows": a few rows of X set to zero, whose
    scale and codes must be zero and whose output must be the bias exactly.
    "+int4": an INT4-only weight image (INT8 matrix cores).  "+g64": the same
    inputs with groups of 64."""
    import torch
    base, _, variant = name.partition("+")
    inp = synth.make(base)
    wl = inp["workload"]
    M, N, K = wl.M, wl.N, wl.K
    g = (64 if variant == "g64" else wl.g) | (REG if variant == "regular" else 0) | (INT4 if variant == "int4" else 0)
    zero_rows = np.array(sorted({1 % M, M // 2, M - 1})) if variant == "zero_rows" else np.array([], int)
    if zero_rows.size:
        inp["x"] = inp["x"].copy()
        inp["x"][zero_rows] = 0
    W = _dev(inp["w"])
    image, sw = gpu.convrot_prepare_weight(W, g)
    ws = gpu.new_workspace(M, K, N, g)
    Y = gpu.convrot_linear(_dev(inp["x"]), image, sw, _dev(inp["bias"]), N, g, workspace=ws)
    Y2 = gpu.convrot_linear(_dev(inp["x"]), image, sw, _dev(inp["bias"]), N, g)
    torch.cuda.synchronize()
    gy = _host_bits(Y)
    assert np.array_equal(gy, _host_bits(Y2)), "two runs differ"
    assert np.all(np.isfinite(synth.bf16_bits_to_f32(gy)))
    og = _oracle_g(g)
    oq_w, osw = oracle.prepare_weight(inp["w"], og)
    y_or, parts = oracle.linear(inp["x"], oq_w, osw, inp["bias"], og, want_parts=True)
    assert np.array_equal(sw.cpu().numpy(), osw), "weight scales"
    wsh = ws.cpu().numpy()
    gq_x = _linear_act_codes(gpu, wsh, M, K, N, g)
    n_x = compare_codes(gq_x, parts["qx"], oracle.rotate_rows(inp["x"], og), parts["sx"], "activation codes")
    qw_all = oracle.unpack_nk(gpu.convrot_host_image_to_nk(image.cpu().numpy(), N, K), K)
    assert qw_all.min() >= -7 and qw_all.max() <= 7
    assert np.all(np.abs(qw_all).max(axis=1) == 7)
    n_w = compare_codes(qw_all, oq_w, oracle.rotate_rows(inp["w"], og), osw, "weight codes")
    rows_ok = np.all(gq_x == parts["qx"], axis=1) & (n_w == 0)
    n_y = compare_y(gy, y_or, rows_ok)
    if zero_rows.size:
        assert np.all(parts["sx"][zero_rows] == 0)
        assert np.all(gq_x[zero_rows] == 0)
        assert np.all(gy[zero_rows] == inp["bias"][None, :]), "zero rows must give the bias"
    print(f"{name}: code mismatches x={n_x} w={n_w}, Y differences {n_y} of {gy.size}")


# --------------------------------------------------------------------------
# ConvRotLinear module: leading dimensions, both paths
# --------------------------------------------------------------------------

@pytest.mark.parametrize("lead,K,N,rotation,path", [((2, 7), 512, 200, "sylvester", "w4a4"),
                                                     ((3, 40), 1024, 96, "regular", "w4a4"),
                                                     ((1, 4), 256, 130, "regular", "w4a16")])
def test_module_matches_the_c_abi(gpu, lead, K, N, rotation, path):
    import torch
    from w4a4_rotated_bit_amd.module import ConvRotLinear
    torch.manual_seed(0)
    lin = torch.nn.Linear(K, N, bias=True).cuda().to(torch.bfloat16)
    mod = ConvRotLinear.from_linear(lin, 256, rotation, path)
    x = torch.randn(*lead, K, device="cuda").to(torch.bfloat16)
    y = mod(x)
    assert y.shape == (*lead, N) and y.dtype == torch.bfloat16
    g = 256 | (REG if rotation == "regular" else 0)
    x2 = x.reshape(-1, K).contiguous()
    fn = gpu.convrot_linear_w4a16 if path == "w4a16" else gpu.convrot_linear
    ref = fn(x2, mod.image, mod.sw, mod.bias, N, g)
    torch.cuda.synchronize()
    assert torch.equal(y.reshape(-1, N), ref)
    # and the oracle agrees on the linear as a whole
    xb = _host_bits(x2)
    wb = _host_bits(lin.weight.detach().contiguous())
    bb = _host_bits(lin.bias.detach().contiguous())
    oq_w, osw = oracle.prepare_weight(wb, g)
    y_or = oracle.linear_w4a16(xb, oq_w, osw, bb, g) if path == "w4a16" else oracle.linear(xb, oq_w, osw, bb, g)
    gy = synth.bf16_bits_to_f32(_host_bits(ref)).astype(np.float64)
    oy = synth.bf16_bits_to_f32(y_or).astype(np.float64)
    assert np.abs(gy - oy).max() <= 1e-2 * np.abs(oy).max()


@pytest.mark.parametrize("rotation", ["sylvester", "regular"])
def test_flux_block_swap(gpu, rotation):
    """Every linear of a small FLUX-shaped block is swapped; the block still
    runs and stays close to the dense block.  The bound is loose on purpose:
    each W4A4 linear alone is about 0.2 off the dense product (relative
    Frobenius), and the residual connections carry the unquantized input."""
    from w4a4_rotated_bit_amd.flux_block import run
    r = run(T=96, hidden=512, group_size=256, rotation=rotation, iters=0)
    print(r)
    assert r["finite"] and r["swapped"] == ["down", "proj", "qkv", "up"]
    assert r["rel_err_update"] < 0.5
    assert r["rel_err_block"] < 0.2


# --------------------------------------------------------------------------
# HIP graph capture: every replay equals the eager result
# --------------------------------------------------------------------------

@pytest.mark.parametrize("M,K,N,g,path", [(1536, 1024, 9216, 256, "w4a4"),     # FP6 256 x 256 tiles
                                          (256, 4096, 256, 256, "w4a4"),       # 192 x 192, split K
                                          (3, 3072, 1000, 256 | REG, "w4a4"),  # one kernel
                                          (40, 1024, 500, 64, "w4a4"),         # prep + INT8 192 x 192
                                          (4, 2048, 700, 256, "w4a16"),        # one kernel
                                          (16, 1024, 300, 64, "w4a16")])       # prep + w4a16_kernel
def test_graph_replays_match_eager(gpu, M, K, N, g, path):
    """The linear captured once into a HIP graph and replayed several times,
    with other work on the GPU in between (another linear on other buffers,
    torch ops, host synchronisations): every replay's Y equals the eager
    result bit for bit (the split-K counters are cleared by a kernel of the
    captured work, not by a memset)."""
    import torch
    x = synth.random_bf16((M, K), seed=M + K + N, outliers=3)
    w = synth.random_bf16((N, K), seed=N + 7, std=0.02)
    b = synth.random_bf16((N,), seed=N + 8, std=0.01)
    X, B = _dev(x), _dev(b)
    image, sw = gpu.convrot_prepare_weight(_dev(w), g)
    fn = gpu.convrot_linear_w4a16 if path == "w4a16" else gpu.convrot_linear
    if path == "w4a16":
        ws = torch.empty(max(gpu.convrot_w4a16_workspace_bytes(M, K, g), 256), dtype=torch.uint8, device="cuda")
    else:
        ws = gpu.new_workspace(M, K, N, g)
    eager = _host_bits(fn(X, image, sw, B, N, g, workspace=ws))
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(X, image, sw, B, N, g, Y=Y, workspace=ws)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn(X, image, sw, B, N, g, Y=Y, workspace=ws)
    other_ws = torch.empty_like(ws)
    for rep in range(4):
        Y.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_host_bits(Y), eager), f"replay {rep}"
        # unrelated eager work between replays, on another workspace
        fn(X, image, sw, B, N, g, workspace=other_ws)
        (X.float() * 2).sum().item()
