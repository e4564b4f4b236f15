"""Seeded synthetic inputs for the ConvRot W4A4 linear.

This module only draws random tensors; it holds none of the method's
arithmetic (no rotation, no quantization, no products).  Both the HIP path's
tests/benchmark and the CPU oracle's checks take their inputs from here.

Shapes follow diffusion-transformer (FLUX-DiT-like) linears: 1024 image + 512
text tokens, hidden size 3072, fused QKV (N = 3 * 3072) and the 4x MLP; plus
the small shapes of the pages' own examples (a 1024 x 1024 weight with a
64-row activation, and the 128 x 2048 by 2048 x 2048 group-64 assay).
Activations are N(0, 1) with a fixed set of outlier channels scaled up (the
structure a rotation is meant to spread out), or GELU of N(0, 1) for an MLP
down-projection input; weights are N(0, 0.02); biases N(0, 0.01) or zero.

Generation: numpy PCG64 streams from ``SeedSequence(seed, spawn_key=(sub,))``
spawned into four children (X, W, bias, outlier channel choice).  Values are
sampled in binary32 and rounded to bf16 (nearest, ties to even).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make", "to_bf16_bits", "bf16_bits_to_f32", "random_bf16"]


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    N: int
    g: int
    seed: int
    sub: int
    x_kind: str            # "normal" or "gelu"
    outlier_count: int     # channels of X scaled by outlier_scale
    outlier_scale: float
    bias_std: float        # 0.0 -> bias of zeros
    w_std: float = 0.02

    @property
    def ops(self) -> int:
        """Integer operations of the product, 2*M*N*K."""
        return 2 * self.M * self.N * self.K

    @property
    def bytes_alg(self) -> int:
        """Bytes the method must move: X bf16, packed INT4 weight, weight
        scales (fp32), bias (bf16) and Y (bf16)."""
        return 2 * self.M * self.K + self.N * self.K // 2 + 4 * self.N + 2 * self.N + 2 * self.M * self.N


def _w(name, M, K, N, g, seed, sub, x_kind, n_out, scale, bias_std):
    return Workload(name, M, K, N, g, seed, sub, x_kind, n_out, scale, bias_std)


# Outlier counts: 8 channels; 1% of 2048 -> 20; 0.5% of 3072 -> 15;
# 1% of 3072 -> 31 (rounded to nearest).
WORKLOADS = {w.name: w for w in [
    _w("tiny_m64_k1024_n1024_g256", 64, 1024, 1024, 256, 1, 0, "normal", 8, 20.0, 0.0),
    _w("g64_m128_k2048_n2048", 128, 2048, 2048, 64, 2, 0, "normal", 20, 20.0, 0.01),
    _w("flux_qkv_m1536_k3072_n9216", 1536, 3072, 9216, 256, 3, 0, "normal", 15, 30.0, 0.01),
    _w("flux_mlp_up_m1536_k3072_n12288", 1536, 3072, 12288, 256, 4, 0, "normal", 0, 1.0, 0.01),
    _w("flux_mlp_down_m1536_k12288_n3072", 1536, 12288, 3072, 256, 4, 1, "gelu", 0, 1.0, 0.01),
    _w("decode_m1_k3072_n12288", 1, 3072, 12288, 256, 5, 0, "normal", 31, 20.0, 0.01),
    _w("decode_m4_k3072_n12288", 4, 3072, 12288, 256, 5, 0, "normal", 31, 20.0, 0.01),
    _w("decode_m16_k3072_n12288", 16, 3072, 12288, 256, 5, 0, "normal", 31, 20.0, 0.01),
    _w("stress_m4096_k3072_n3072", 4096, 3072, 3072, 256, 5, 1, "normal", 31, 20.0, 0.01),
]}


def to_bf16_bits(a) -> np.ndarray:
    """binary32 -> bf16 bit patterns, nearest-even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _streams(seed: int, sub: int):
    ss = np.random.SeedSequence(entropy=seed, spawn_key=(sub,))
    return [np.random.Generator(np.random.PCG64(c)) for c in ss.spawn(4)]


def _gelu(z: np.ndarray) -> np.ndarray:
    from scipy.special import erf
    z64 = z.astype(np.float64)
    return (0.5 * z64 * (1.0 + erf(z64 / np.sqrt(2.0)))).astype(np.float32)


def make(name_or_wl, M: int | None = None, with_weight: bool = True):
    """Build the seeded inputs of a workload.

    Returns a dict with bf16 bit arrays ``x`` [M, K], ``w`` [N, K] (if
    ``with_weight``), ``bias`` [N] (zeros when the recipe says so) and the
    workload record.  ``M`` overrides the row count (rows are a prefix of the
    same stream, so a smaller M gives the leading rows of a larger one)."""
    wl = WORKLOADS[name_or_wl] if isinstance(name_or_wl, str) else name_or_wl
    rows = wl.M if M is None else int(M)
    gx, gw, gb, go = _streams(wl.seed, wl.sub)
    z = gx.standard_normal((rows, wl.K), dtype=np.float32)
    if wl.x_kind == "gelu":
        x = _gelu(z)
    else:
        x = z
        if wl.outlier_count:
            idx = go.choice(wl.K, size=wl.outlier_count, replace=False)
            x[:, idx] *= np.float32(wl.outlier_scale)
    out = {"workload": wl, "x": to_bf16_bits(x)}
    if with_weight:
        w = gw.standard_normal((wl.N, wl.K), dtype=np.float32) * np.float32(wl.w_std)
        out["w"] = to_bf16_bits(w)
    if wl.bias_std > 0:
        out["bias"] = to_bf16_bits(gb.standard_normal((wl.N,), dtype=np.float32) * np.float32(wl.bias_std))
    else:
        out["bias"] = np.zeros((wl.N,), dtype=np.uint16)
    return out


def random_bf16(shape, seed: int, std: float = 1.0, outliers: int = 0, outlier_scale: float = 20.0) -> np.ndarray:
    """Generic seeded bf16 matrix for edge-case tests: N(0, std) with optional
    outlier columns."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=seed, spawn_key=(99,))))
    a = rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
    if outliers and len(shape) == 2:
        idx = rng.choice(shape[1], size=min(outliers, shape[1]), replace=False)
        a[:, idx] *= np.float32(outlier_scale)
    return to_bf16_bits(a)
