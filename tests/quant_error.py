"""Quantization error of the W4A4 linear against the dense product.

For each workload, runs ``convrot_linear`` on the GPU with the Sylvester and
with the regular Hadamard rotation, and compares Y with the dense
Y_ref = X W^T + bias (binary64, from the bf16 inputs) on a sample of rows.
As a point of reference it also reports rowwise absmax INT4 quantization of
X and W without any rotation, quantized by the oracle's quantizer (the same
rule: s = absmax / 7, codes clamp(rint(v / s), -7, 7)).  A measurement
script beside the tests (it reads the oracle, so it stays out of the
package).

Usage: python tests/quant_error.py [workload ...]
Prints one JSON line per workload.
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import oracle  # noqa: E402
from w4a4_rotated_bit_amd import binding, synth  # noqa: E402


def _rowwise_int4(a: np.ndarray):
    """Rowwise absmax INT4 codes and scales of binary32 rows, by the oracle."""
    q, s = oracle.quantize_rows(a.astype(np.float32))
    return q.astype(np.float64), s.astype(np.float64)[:, None]


def _errors(y: np.ndarray, ref: np.ndarray) -> dict:
    d = y - ref
    return {"rel_fro": float(np.linalg.norm(d) / np.linalg.norm(ref)),
            "max_abs_over_rms": float(np.abs(d).max() / np.sqrt(np.mean(ref ** 2)))}


def report(name: str, rows: int = 64, seed: int = 7) -> dict:
    import torch
    inp = synth.make(name)
    wl = inp["workload"]
    M, N, K = wl.M, wl.N, wl.K
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    X, W, B = dev(inp["x"]), dev(inp["w"]), dev(inp["bias"])
    pick = np.sort(np.random.default_rng(seed).choice(M, size=min(rows, M), replace=False))
    xf = synth.bf16_bits_to_f32(inp["x"][pick]).astype(np.float64)
    wf = synth.bf16_bits_to_f32(inp["w"]).astype(np.float64)
    bf = synth.bf16_bits_to_f32(inp["bias"]).astype(np.float64)
    ref = xf @ wf.T + bf[None, :]
    out = {"workload": name, "M": M, "K": K, "N": N, "group": wl.g, "rows_sampled": int(len(pick))}
    for label, flag in (("sylvester", 0), ("regular", binding.CONVROT_REGULAR_HADAMARD)):
        image, sw = binding.convrot_prepare_weight(W, wl.g | flag)
        Y = binding.convrot_linear(X, image, sw, B, N, wl.g | flag)
        torch.cuda.synchronize()
        y = Y.float().cpu().numpy().astype(np.float64)[pick]
        out[label] = _errors(y, ref)
    qx, sx = _rowwise_int4(xf)
    qw, swn = _rowwise_int4(wf)
    out["no_rotation"] = _errors((qx @ qw.T) * sx * swn.T + bf[None, :], ref)
    return out


def main(argv: list[str]) -> int:
    binding.load()
    names = argv or list(synth.WORKLOADS)
    for name in names:
        print(json.dumps(report(name)), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
