"""The allocation-free linear (convrot_linear_noalloc, for callers that cannot
allocate device memory) against convrot_linear, the entry point it is a
variant of: identical Y, bit for bit, on calls in a row whose inputs shrink
(the library's workspace keeps the previous call's contents), on every kernel
path (FP6 and INT8 block tiles, split K, the one-kernel small-M path), and a
clear error for a shape whose workspace exceeds the library's array."""
import numpy as np
import pytest

from w4a4_rotated_bit_amd import synth

pytestmark = pytest.mark.gpu

REG = 0x10000
INT4 = 0x20000


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


# largest first: every later call runs on a workspace holding a larger call's data
CALLS = [(1536, 12288, 3072, 256),        # INT8 192 x 192, K split 2 ways (partial tiles, counters)
         (1536, 3072, 9216, 256),         # FP6 256 x 256
         (300, 1024, 700, 64 | REG),      # INT8 192 x 192, unsplit
         (256, 4096, 256, 256),           # split again, smaller
         (40, 1000, 300, 256 | INT4),     # INT4 image, ragged K
         (16, 3072, 1000, 256),           # weight streaming
         (3, 3072, 1000, 256 | REG)]      # one kernel


def test_noalloc_linear_matches_linear_on_shrinking_calls(gpu):
    import torch
    for i, (M, K, N, g) in enumerate(CALLS):
        x = synth.random_bf16((M, K), seed=M + K + i, outliers=3)
        w = synth.random_bf16((N, K), seed=N + 11 * i, std=0.02)
        b = synth.random_bf16((N,), seed=N + i, std=0.01)
        X, B = _dev(x), _dev(b)
        image, sw = gpu.convrot_prepare_weight(_dev(w), g)
        ref = gpu.convrot_linear(X, image, sw, B, N, g)
        Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        gpu.convrot_linear_noalloc(X, image, sw, B, N, g, Y)
        Y2 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        gpu.convrot_linear_noalloc(X, image, sw, None if i % 2 else B, N, g, Y2)   # twice in a row, bias or not
        ref2 = gpu.convrot_linear(X, image, sw, None if i % 2 else B, N, g)
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), ref.view(torch.int16)), (M, K, N, g)
        assert torch.equal(Y2.view(torch.int16), ref2.view(torch.int16)), (M, K, N, g)


def test_noalloc_linear_rejects_shapes_beyond_its_workspace(gpu):
    import torch
    M, K, N, g = 4096, 16384, 256, 256
    assert gpu.convrot_workspace_bytes(M, K, N, g) > gpu.NOALLOC_MAX_WORKSPACE
    X = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    image = torch.zeros(gpu.convrot_weight_image_bytes(N, K, g), dtype=torch.uint8, device="cuda")
    sw = torch.zeros(N, dtype=torch.float32, device="cuda")
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gpu.ConvRotError) as e:
        gpu.convrot_linear_noalloc(X, image, sw, None, N, g, Y)
    assert e.value.status == gpu.CONVROT_EWORKSPACE
