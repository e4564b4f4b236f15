"""ConvRotLinear: a torch module around the library's W4A4 (or W4A16) linear.

The weight is rotated, quantized and packed once, on construction from an
``nn.Linear`` (the offline step; convrot-mlx README, "What is included": the
conversion of eligible linears and the ConvRotLinear layer that replaces
them).  ``forward`` flattens the leading dimensions of x to M rows, runs
``convrot_linear`` (or ``convrot_linear_w4a16``) on the current stream and
restores them.  Every step of the linear runs in the library's kernels; the
module only holds buffers and reshapes.
"""
from __future__ import annotations

import torch

from . import binding


class ConvRotLinear(torch.nn.Module):
    """y = x W^T + b with the ConvRot rotation and INT4 weights.

    group_size: 64 or 256; rotation: "sylvester" or "regular"; path: "w4a4"
    (activations quantized to INT4) or "w4a16" (bf16 rotated activations,
    M <= 32 rows per call)."""

    def __init__(self, in_features: int, out_features: int, image: torch.Tensor, sw: torch.Tensor,
                 bias: torch.Tensor | None, group_size: int = 256, rotation: str = "sylvester", path: str = "w4a4"):
        super().__init__()
        if rotation not in ("sylvester", "regular"):
            raise ValueError(f"unknown rotation {rotation!r}")
        if path not in ("w4a4", "w4a16"):
            raise ValueError(f"unknown path {path!r}")
        self.in_features, self.out_features = in_features, out_features
        self.group_size, self.rotation, self.path = group_size, rotation, path
        self.g = group_size | (binding.CONVROT_REGULAR_HADAMARD if rotation == "regular" else 0)
        self.register_buffer("image", image)
        self.register_buffer("sw", sw)
        self.register_buffer("bias", bias)

    @classmethod
    @torch.no_grad()
    def from_linear(cls, linear: torch.nn.Linear, group_size: int = 256, rotation: str = "sylvester",
                    path: str = "w4a4") -> "ConvRotLinear":
        if not linear.weight.is_cuda:
            raise ValueError("the linear must be on the GPU")
        w = linear.weight.detach().to(torch.bfloat16).contiguous()
        g = group_size | (binding.CONVROT_REGULAR_HADAMARD if rotation == "regular" else 0)
        image, sw = binding.convrot_prepare_weight(w, g)
        b = None if linear.bias is None else linear.bias.detach().to(torch.bfloat16).contiguous()
        return cls(linear.in_features, linear.out_features, image, sw, b, group_size, rotation, path)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if x.shape[-1] != self.in_features:
            raise ValueError(f"last dimension {x.shape[-1]} != in_features {self.in_features}")
        lead = x.shape[:-1]
        x2 = x.reshape(-1, self.in_features).to(torch.bfloat16).contiguous()
        if self.path == "w4a16":
            y = binding.convrot_linear_w4a16(x2, self.image, self.sw, self.bias, self.out_features, self.g)
        else:
            y = binding.convrot_linear(x2, self.image, self.sw, self.bias, self.out_features, self.g)
        return y.reshape(*lead, self.out_features)

    def extra_repr(self) -> str:
        return (f"in_features={self.in_features}, out_features={self.out_features}, bias={self.bias is not None}, "
                f"group_size={self.group_size}, rotation={self.rotation}, path={self.path}")


def eligible(linear: torch.nn.Linear, group_size: int = 256) -> bool:
    """Whether the library takes this linear: K a multiple of 8 whose rotated
    width fits, and N within the row limit."""
    K, N = linear.in_features, linear.out_features
    return K % 8 == 0 and binding.rotated_width(K, group_size) <= binding.MAX_K and 1 <= N <= binding.MAX_ROWS


@torch.no_grad()
def convert_linears(model: torch.nn.Module, group_size: int = 256, rotation: str = "sylvester", path: str = "w4a4",
                    include=None) -> list[str]:
    """Replace, in place, every eligible ``nn.Linear`` of ``model`` (and whose
    qualified name ``include(name)`` accepts, when given) by a ConvRotLinear
    built from it -- the module swap of the convrot-mlx README, "What is
    included".  Returns the names of the replaced linears."""
    done = []
    for name, parent in list(model.named_modules()):
        for child_name, child in list(parent.named_children()):
            full = f"{name}.{child_name}" if name else child_name
            if type(child) is not torch.nn.Linear or not eligible(child, group_size):
                continue
            if include is not None and not include(full):
                continue
            setattr(parent, child_name, ConvRotLinear.from_linear(child, group_size, rotation, path))
            done.append(full)
    return done
