"""A synthetic FLUX-shaped transformer block, run dense and with its linears
swapped for ConvRotLinear.

The pages measure ConvRot inside FLUX.1 Dev image generation (convrot-mlx
README, "Why this repository exists"); no FLUX weights, prompts or runtime are
used here.  This harness builds one block of the same shape with random
weights (N(0, 0.02), biases N(0, 0.01)) and synthetic tokens (N(0, 1) with a
few outlier channels scaled up), and runs it twice: with plain bf16
``nn.Linear`` layers, and after ``convert_linears`` has replaced every linear
by a ConvRotLinear (the module swap of the convrot-mlx README, "What is
included").  It reports the relative Frobenius error of the block output and
the time per block of both.

Block, hidden size H, heads of 128, T tokens:
    h = LayerNorm(x) * (1 + scale) + shift       (random modulation)
    q, k, v = qkv(h)                             H -> 3H
    x = x + proj(softmax(q k^T / sqrt(128)) v)   H -> H
    x = x + down(gelu_tanh(up(LayerNorm(x))))    H -> 4H -> H
The norms and the attention run in float32 torch ops around the linears;
they are the harness, not the path.

    python -m w4a4_rotated_bit_amd.flux_block [--tokens 1536] [--hidden 3072]
        [--rotation sylvester|regular] [--group-size 256] [--iters 20]
"""
from __future__ import annotations

import argparse
import copy
import json
import sys

import torch

from . import synth
from .module import ConvRotLinear, convert_linears


class Block(torch.nn.Module):
    def __init__(self, hidden: int, head_dim: int = 128, seed: int = 0):
        super().__init__()
        if hidden % head_dim:
            raise ValueError("hidden must be a multiple of the head size")
        self.hidden, self.head_dim, self.heads = hidden, head_dim, hidden // head_dim
        self.qkv = torch.nn.Linear(hidden, 3 * hidden)
        self.proj = torch.nn.Linear(hidden, hidden)
        self.up = torch.nn.Linear(hidden, 4 * hidden)
        self.down = torch.nn.Linear(4 * hidden, hidden)
        for i, lin in enumerate((self.qkv, self.proj, self.up, self.down)):
            n, k = lin.weight.shape
            w = synth.random_bf16((n, k), seed=seed * 16 + 2 * i, std=0.02)
            b = synth.random_bf16((n,), seed=seed * 16 + 2 * i + 1, std=0.01)
            lin.weight.data = torch.from_numpy(synth.bf16_bits_to_f32(w)).to(torch.bfloat16)
            lin.bias.data = torch.from_numpy(synth.bf16_bits_to_f32(b)).to(torch.bfloat16)
        mod = synth.random_bf16((2, hidden), seed=seed * 16 + 9, std=0.1)
        self.register_buffer("modulation", torch.from_numpy(synth.bf16_bits_to_f32(mod)))

    @staticmethod
    def _norm(x: torch.Tensor) -> torch.Tensor:
        return torch.nn.functional.layer_norm(x.float(), (x.shape[-1],), eps=1e-6)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        """x: bf16 [T, hidden] -> bf16 [T, hidden]."""
        T, H = x.shape
        shift, scale = self.modulation[0], self.modulation[1]
        h = (self._norm(x) * (1 + scale) + shift).to(torch.bfloat16)
        qkv = self.qkv(h).float().reshape(T, 3, self.heads, self.head_dim)
        q, k, v = (qkv[:, i].transpose(0, 1).contiguous() for i in range(3))   # [heads, T, D] each
        s = torch.bmm(q, k.transpose(1, 2).contiguous()) / self.head_dim ** 0.5
        a = torch.bmm(torch.softmax(s, dim=-1), v).transpose(0, 1).reshape(T, H)
        x = (x.float() + self.proj(a.to(torch.bfloat16)).float()).to(torch.bfloat16)
        u = torch.nn.functional.gelu(self.up(self._norm(x).to(torch.bfloat16)).float(), approximate="tanh")
        return (x.float() + self.down(u.to(torch.bfloat16)).float()).to(torch.bfloat16)


def tokens(T: int, hidden: int, seed: int = 7) -> torch.Tensor:
    """Synthetic bf16 tokens: N(0, 1), 1% of the channels scaled by 20."""
    bits = synth.random_bf16((T, hidden), seed=seed, outliers=max(1, round(0.01 * hidden)))
    return torch.from_numpy(synth.bf16_bits_to_f32(bits)).to(torch.bfloat16)


def rel_err(y: torch.Tensor, ref: torch.Tensor) -> float:
    y, ref = y.detach().double(), ref.detach().double()
    return float(torch.linalg.vector_norm(y - ref) / torch.linalg.vector_norm(ref))


def time_ms(fn, x: torch.Tensor, iters: int) -> float:
    for _ in range(3):
        fn(x)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(iters):
        fn(x)
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / iters


@torch.no_grad()
def run(T: int = 1536, hidden: int = 3072, group_size: int = 256, rotation: str = "sylvester",
        iters: int = 20) -> dict:
    dense = Block(hidden).cuda().to(torch.bfloat16)
    dense.modulation = dense.modulation.float()
    quant = copy.deepcopy(dense)
    swapped = convert_linears(quant, group_size, rotation)
    if sorted(swapped) != ["down", "proj", "qkv", "up"]:
        raise RuntimeError(f"unexpected linears swapped: {swapped}")
    assert all(isinstance(getattr(quant, n), ConvRotLinear) for n in swapped)
    x = tokens(T, hidden).cuda()
    y_dense, y_quant = dense(x), quant(x)
    torch.cuda.synchronize()
    out = {
        "tokens": T, "hidden": hidden, "group_size": group_size, "rotation": rotation,
        "swapped": sorted(swapped),
        "rel_err_block": rel_err(y_quant, y_dense),
        "rel_err_update": rel_err(y_quant.float() - x.float(), y_dense.float() - x.float()),
        "finite": bool(torch.isfinite(y_quant.float()).all()),
    }
    if iters > 0:
        out["dense_ms"] = time_ms(dense, x, iters)
        out["convrot_ms"] = time_ms(quant, x, iters)
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--tokens", type=int, default=1536)
    ap.add_argument("--hidden", type=int, default=3072)
    ap.add_argument("--group-size", type=int, default=256, choices=(64, 256))
    ap.add_argument("--rotation", default="sylvester", choices=("sylvester", "regular"))
    ap.add_argument("--iters", type=int, default=20)
    args = ap.parse_args(argv)
    if not torch.cuda.is_available():
        print("a GPU is required", file=sys.stderr)
        return 2
    print(json.dumps(run(args.tokens, args.hidden, args.group_size, args.rotation, args.iters)))
    return 0


if __name__ == "__main__":
    sys.exit(main())
