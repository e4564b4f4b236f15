"""ConvRot W4A4 rotated linear for AMD Instinct MI355X (gfx950).

The compute path is a C-ABI shared library of hand-written HIP kernels
(``csrc/``, declared in ``include/convrot.h``); ``binding`` is its thin ctypes
binding (PyTorch supplies device memory and streams).  ``synth`` draws the
seeded synthetic inputs.  Importing the package loads nothing native; the
library is loaded on first use and its absence is an error, never a fallback.
"""
__all__ = ["binding", "synth"]
