"""Host-side checks of the torch module layer: which linears the swap takes,
and the FLUX-shaped block harness's own shapes (dense, on the CPU)."""
import pytest
import torch

from w4a4_rotated_bit_amd import binding
from w4a4_rotated_bit_amd.flux_block import Block, rel_err, tokens
from w4a4_rotated_bit_amd.module import eligible


@pytest.mark.parametrize("K,N,ok", [(1024, 64, True), (1000, 64, True), (1001, 64, False), (8, 1, True),
                                    (binding.MAX_K, 3, True), (binding.MAX_K + 8, 3, False)])
def test_eligible(K, N, ok):
    lin = torch.nn.Linear(K, N, bias=False, device="meta")
    assert eligible(lin, 256) is ok


def test_block_shapes_on_cpu():
    blk = Block(256, head_dim=64).to(torch.bfloat16)
    blk.modulation = blk.modulation.float()
    x = tokens(40, 256)
    y = blk(x)
    assert y.shape == x.shape and y.dtype == torch.bfloat16
    assert torch.isfinite(y.float()).all()
    assert rel_err(y, y) == 0.0
    assert 0.0 < rel_err(y, x) < 1.0       # the block adds an update to its input
