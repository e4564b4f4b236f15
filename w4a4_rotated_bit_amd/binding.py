"""Thin ctypes binding of libconvrot.so (the C ABI in include/convrot.h).

Argument marshalling only: every step of the ConvRot path runs in the HIP
kernels behind the C ABI.  PyTorch provides device memory (output tensors are
allocated with ``torch.empty``) and the stream (torch's current stream).
Function names are those of the C ABI.  A non-zero status raises
``ConvRotError``; a missing library raises at load time -- there is no
fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np

from . import build as _build

LIB_PATH = _build.LIB_PATH

CONVROT_OK = 0
CONVROT_EINVAL = 1
CONVROT_EWORKSPACE = 2
CONVROT_EHIP = 3
CONVROT_EDEVICE = 4
# OR'd into a group size g: rotate with the regular Hadamard matrix
CONVROT_REGULAR_HADAMARD = 0x10000
# OR'd into a group size g: the weight image holds the INT4 codes only (0.5 bytes
# per weight); every product then runs on the INT8 matrix cores
CONVROT_INT4_IMAGE = 0x20000
_GROUP_FLAGS = CONVROT_REGULAR_HADAMARD | CONVROT_INT4_IMAGE
# workspace status word: offset, and the value a split-K wait that ran out leaves
WORKSPACE_STATUS_OFFSET = 2048
CONVROT_STATUS_SPLIT_TIMEOUT = 1
# test flag of convrot_gemm_i32_tiled
CONVROT_TEST_SPLIT_TIMEOUT = 1
CONVROT_TILE_FP6 = 0x10000  # or-ed into tile_n of the tiled hooks: the FP6 tile of that size (192 x 384)
MAX_K = 16384           # largest rotated width K_rot
MAX_ROWS = 16777216     # largest M or N


def rotated_width(K: int, g: int) -> int:
    """Codes and rotated values are K rounded up to a whole number of groups wide
    (the missing values of the last group are zero)."""
    gs = g & ~_GROUP_FLAGS
    return -(-K // gs) * gs

_lock = threading.Lock()
_lib = None


class ConvRotError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        text = _lib.convrot_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{where}: status {status} ({text})")


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "convrot_status_string": ([_I], ctypes.c_char_p),
    "convrot_version": ([], ctypes.c_char_p),
    "convrot_weight_image_bytes": ([_I64, _I64, _I, ctypes.POINTER(_SZ)], _I),
    "convrot_workspace_bytes": ([_I64, _I64, _I64, _I, ctypes.POINTER(_SZ)], _I),
    "convrot_linear_kernel_count": ([_I64, _I64, _I64, _I, ctypes.POINTER(_I)], _I),
    "convrot_linear_plan": ([_I64, _I64, _I64, _I] + [ctypes.POINTER(_I)] * 4, _I),
    "convrot_validate_weight": ([_P, _I64, _I64, _I, _P, _P], _I),
    "convrot_validate_linear": ([_P, _I64, _I64, _P, _P, _P, _I64, _I, _P, _P, _SZ], _I),
    "convrot_prepare_weight": ([_P, _I64, _I64, _I, _P, _P, _P], _I),
    "convrot_quantize_weight": ([_P, _I64, _I64, _I, _P, _P, _P], _I),
    "convrot_repack_nk_to_image": ([_P, _I64, _I64, _I, _P, _P], _I),
    "convrot_linear": ([_P, _I64, _I64, _P, _P, _P, _I64, _I, _P, _P, _SZ, _P], _I),
    "convrot_linear_noalloc": ([_P, _I64, _I64, _P, _P, _P, _I64, _I, _P, _P], _I),
    "convrot_prepare_activations": ([_P, _I64, _I64, _I, _P, _SZ, _P], _I),
    "convrot_gemm": ([_P, _SZ, _I64, _I64, _P, _P, _P, _I64, _I, _P, _P], _I),
    "convrot_prepare_rows": ([_P, _I64, _I64, _I, _P, _P, _P, _P], _I),
    "convrot_w4a16_workspace_bytes": ([_I64, _I64, _I, _P], _I),
    "convrot_validate_linear_w4a16": ([_P, _I64, _I64, _P, _P, _P, _I64, _I, _P, _P, _SZ], _I),
    "convrot_linear_w4a16": ([_P, _I64, _I64, _P, _P, _P, _I64, _I, _P, _P, _SZ, _P], _I),
    "convrot_gemm_i32": ([_P, _I64, _I64, _P, _I64, _P, _P, _SZ, _P], _I),
    "convrot_workspace_bytes_tiled": ([_I64, _I64, _I64, _I, _I, _I, ctypes.POINTER(_SZ)], _I),
    "convrot_gemm_i32_tiled": ([_P, _I64, _I64, _P, _I64, _P, _I, _I, _I, _I, _P, _SZ, _P], _I),
    "convrot_split_k_extent": ([_I64, _I64, _I64, _I, _I, _I, ctypes.POINTER(_SZ), ctypes.POINTER(_I),
                                ctypes.POINTER(_SZ)], _I),
    "convrot_matrix_core_probe_bytes": ([ctypes.POINTER(_SZ)], _I),
    "convrot_matrix_core_probe": ([_I, _I, _P, _SZ, ctypes.POINTER(_I64), _P], _I),
    "convrot_host_pack_nk": ([_P, _I64, _I64, _P], _I),
    "convrot_host_unpack_nk": ([_P, _I64, _I64, _P], _I),
    "convrot_host_nk_to_kn": ([_P, _I64, _I64, _P], _I),
    "convrot_host_kn_to_nk": ([_P, _I64, _I64, _P], _I),
    "convrot_host_nk_to_image": ([_P, _I64, _I64, _P], _I),
    "convrot_host_image_to_nk": ([_P, _I64, _I64, _P], _I),
    "convrot_host_act_image_to_codes": ([_P, _I64, _I64, _P], _I),
    "convrot_host_image_fp6_to_nk": ([_P, _I64, _I64, _P], _I),
    "convrot_host_workspace_fp6_codes": ([_P, _I64, _I64, _P], _I),
}


def load():
    """Load libconvrot.so (building it only if nothing is built).

    torch is imported first: it brings its own HIP runtime library, and the
    library's HIP dependency must resolve to that same, already loaded copy --
    loaded the other way round, the process would hold two HIP runtimes and
    torch's device pointers and streams would be foreign to the library's."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        import torch  # noqa: F401  (see above)
        if not os.path.exists(LIB_PATH):
            _build.build()
        lib = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
        return lib


def _call(name, *args):
    rc = getattr(load(), name)(*args)
    if rc != CONVROT_OK:
        raise ConvRotError(rc, name)


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t, dtype, name):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


# --------------------------------------------------------------------------
# sizes and checks
# --------------------------------------------------------------------------

def convrot_version() -> str:
    return load().convrot_version().decode()


def convrot_status_string(status: int) -> str:
    return load().convrot_status_string(int(status)).decode()


def convrot_weight_image_bytes(N: int, K: int, g: int) -> int:
    out = _SZ(0)
    _call("convrot_weight_image_bytes", N, K, g, ctypes.byref(out))
    return out.value


def convrot_workspace_bytes(M: int, K: int, N: int, g: int) -> int:
    out = _SZ(0)
    _call("convrot_workspace_bytes", M, K, N, g, ctypes.byref(out))
    return out.value


def convrot_linear_kernel_count(M: int, K: int, N: int, g: int) -> int:
    out = _I(0)
    _call("convrot_linear_kernel_count", M, K, N, g, ctypes.byref(out))
    return out.value


CONVROT_MFMA_I8 = 1
CONVROT_MFMA_FP6 = 2


def convrot_linear_plan(M: int, K: int, N: int, g: int) -> dict:
    """The product plan: {"mfma": CONVROT_MFMA_I8 / CONVROT_MFMA_FP6 (0 if M or N
    is 0), "tile": (tile_m, tile_n) ((0, 0) for M <= 128), "splits": S}."""
    v = [ctypes.c_int() for _ in range(4)]
    _call("convrot_linear_plan", M, K, N, g, *[ctypes.byref(x) for x in v])
    return {"mfma": v[0].value, "tile": (v[1].value, v[2].value), "splits": v[3].value}


def convrot_validate_weight(W_ptr, N, K, g, image_ptr, sw_ptr) -> int:
    """Raw pointer values (ints); returns the status code."""
    return load().convrot_validate_weight(W_ptr, N, K, g, image_ptr, sw_ptr)


def convrot_validate_linear(X_ptr, M, K, image_ptr, sw_ptr, bias_ptr, N, g, Y_ptr, ws_ptr, ws_bytes) -> int:
    """Raw pointer values (ints); returns the status code."""
    return load().convrot_validate_linear(X_ptr, M, K, image_ptr, sw_ptr, bias_ptr, N, g, Y_ptr, ws_ptr, ws_bytes)


# --------------------------------------------------------------------------
# device entry points
# --------------------------------------------------------------------------

def convrot_prepare_weight(W, g: int, image=None, sw=None, stream=None):
    """W: bf16 [N, K] on the GPU -> (weight image uint8, sw float32 [N])."""
    import torch
    N, K = W.shape
    nbytes = convrot_weight_image_bytes(N, K, g)
    if image is None:
        image = torch.empty(nbytes, dtype=torch.uint8, device=W.device)
    if sw is None:
        sw = torch.empty(N, dtype=torch.float32, device=W.device)
    if image.numel() < nbytes:
        raise ValueError("weight image buffer too small")
    _call("convrot_prepare_weight", _dev(W, torch.bfloat16, "W"), N, K, g, _dev(image, torch.uint8, "image"),
          _dev(sw, torch.float32, "sw"), _stream(stream))
    return image, sw


def convrot_quantize_weight(W, g: int, stream=None):
    """W: bf16 [N, K] -> (N x packed-K uint8 [N, K_rot/2], sw float32 [N]), K_rot = rotated_width(K, g)."""
    import torch
    N, K = W.shape
    nk = torch.empty((N, rotated_width(K, g) // 2), dtype=torch.uint8, device=W.device)
    sw = torch.empty(N, dtype=torch.float32, device=W.device)
    _call("convrot_quantize_weight", _dev(W, torch.bfloat16, "W"), N, K, g, _dev(nk, torch.uint8, "nk"),
          _dev(sw, torch.float32, "sw"), _stream(stream))
    return nk, sw


def convrot_repack_nk_to_image(nk, N: int, K: int, g: int = 64, stream=None):
    """N x packed-K uint8 [N, K_rot/2] -> weight image (the FP6 copy too unless g has CONVROT_INT4_IMAGE)."""
    import torch
    image = torch.empty(convrot_weight_image_bytes(N, K, g), dtype=torch.uint8, device=nk.device)
    _call("convrot_repack_nk_to_image", _dev(nk, torch.uint8, "nk"), N, K, g, _dev(image, torch.uint8, "image"),
          _stream(stream))
    return image


def new_workspace(M: int, K: int, N: int, g: int, device="cuda"):
    import torch
    return torch.empty(convrot_workspace_bytes(M, K, N, g), dtype=torch.uint8, device=device)


def convrot_linear(X, image, sw, bias, N: int, g: int, Y=None, workspace=None, stream=None):
    """X: bf16 [M, K]; bias: bf16 [N] or None -> Y bf16 [M, N]."""
    import torch
    M, K = X.shape
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    if workspace is None:
        workspace = new_workspace(M, K, N, g, X.device)
    bias_p = None if bias is None else _dev(bias, torch.bfloat16, "bias")
    _call("convrot_linear", _dev(X, torch.bfloat16, "X"), M, K, _dev(image, torch.uint8, "image"),
          _dev(sw, torch.float32, "sw"), bias_p, N, g, _dev(Y, torch.bfloat16, "Y"),
          _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream))
    return Y


# the largest workspace convrot_linear_noalloc has (CONVROT_NOALLOC_MAX_WORKSPACE)
NOALLOC_MAX_WORKSPACE = 48 << 20


def convrot_linear_noalloc(X, image, sw, bias, N: int, g: int, Y, stream=None):
    """convrot_linear with the library's own device workspace (no allocation in
    the call; Y must be given).  Calls on one GPU share that workspace."""
    import torch
    M, K = X.shape
    bias_p = None if bias is None else _dev(bias, torch.bfloat16, "bias")
    _call("convrot_linear_noalloc", _dev(X, torch.bfloat16, "X"), M, K, _dev(image, torch.uint8, "image"),
          _dev(sw, torch.float32, "sw"), bias_p, N, g, _dev(Y, torch.bfloat16, "Y"), _stream(stream))
    return Y


def convrot_prepare_activations(X, g: int, workspace, stream=None):
    import torch
    M, K = X.shape
    _call("convrot_prepare_activations", _dev(X, torch.bfloat16, "X"), M, K, g,
          _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream))
    return workspace


def convrot_gemm(workspace, M: int, K: int, image, sw, bias, N: int, g: int, Y=None, stream=None):
    """The GEMM half of convrot_linear (M, K, N, g as for the linear) on a prepared workspace."""
    import torch
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=workspace.device)
    bias_p = None if bias is None else _dev(bias, torch.bfloat16, "bias")
    _call("convrot_gemm", _dev(workspace, torch.uint8, "workspace"), workspace.numel(), M, K,
          _dev(image, torch.uint8, "image"), _dev(sw, torch.float32, "sw"), bias_p, N, g,
          _dev(Y, torch.bfloat16, "Y"), _stream(stream))
    return Y


def convrot_prepare_rows(X, g: int, want_rotated: bool = False, stream=None):
    """Rotation + quantization of bf16 rows -> (codes int8 [rows, K_rot], scales f32 [rows],
    rotated f32 [rows, K_rot] or None), K_rot = rotated_width(K, g)."""
    import torch
    rows, K = X.shape
    Kr = rotated_width(K, g)
    codes = torch.empty((rows, Kr), dtype=torch.int8, device=X.device)
    scales = torch.empty(rows, dtype=torch.float32, device=X.device)
    rot = torch.empty((rows, Kr), dtype=torch.float32, device=X.device) if want_rotated else None
    _call("convrot_prepare_rows", _dev(X, torch.bfloat16, "X"), rows, K, g, _dev(codes, torch.int8, "codes"),
          _dev(scales, torch.float32, "scales"), None if rot is None else _dev(rot, torch.float32, "rotated"),
          _stream(stream))
    return codes, scales, rot


def convrot_gemm_i32(qx, image, N: int, workspace=None, stream=None):
    """qx: int8 codes [M, K] -> int32 [M, N] products against the weight image."""
    import torch
    M, K = qx.shape
    if workspace is None:
        workspace = new_workspace(M, K, N, 64, qx.device)
    acc = torch.empty((M, N), dtype=torch.int32, device=qx.device)
    _call("convrot_gemm_i32", _dev(qx, torch.int8, "qx"), M, K, _dev(image, torch.uint8, "image"), N,
          _dev(acc, torch.int32, "acc"), _dev(workspace, torch.uint8, "workspace"), workspace.numel(),
          _stream(stream))
    return acc


def convrot_workspace_bytes_tiled(M: int, K: int, N: int, tile, splits: int) -> int:
    out = _SZ(0)
    _call("convrot_workspace_bytes_tiled", M, K, N, tile[0], tile[1], splits, ctypes.byref(out))
    return out.value


def convrot_gemm_i32_tiled(qx, image, N: int, tile, splits: int, test_flags: int = 0, workspace=None, stream=None):
    """convrot_gemm_i32 with the block tile (tile_m, tile_n) and the K split given
    (tile_n | CONVROT_TILE_FP6 picks the FP6 192 x 384 tile over the INT8 one).
    Returns (acc int32 [M, N], workspace)."""
    import torch
    M, K = qx.shape
    if workspace is None:
        workspace = torch.empty(convrot_workspace_bytes_tiled(M, K, N, tile, splits), dtype=torch.uint8,
                                device=qx.device)
    acc = torch.empty((M, N), dtype=torch.int32, device=qx.device)
    _call("convrot_gemm_i32_tiled", _dev(qx, torch.int8, "qx"), M, K, _dev(image, torch.uint8, "image"), N,
          _dev(acc, torch.int32, "acc"), tile[0], tile[1], splits, test_flags,
          _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream))
    return acc, workspace


def convrot_split_k_extent(M: int, K: int, N: int, tile, splits: int) -> dict:
    """Host check of a split-K plan's footprint: one past the largest partial-area
    byte, counter word and LDS byte the exchange touches."""
    pe, cu, le = _SZ(0), _I(0), _SZ(0)
    _call("convrot_split_k_extent", M, K, N, tile[0], tile[1], splits, ctypes.byref(pe), ctypes.byref(cu),
          ctypes.byref(le))
    return {"partial_end": pe.value, "counters_used": cu.value, "lds_end": le.value}


CONVROT_PROBE_FP6 = 1
CONVROT_PROBE_INT8 = 2
PROBE_OPS_PER_MFMA = {CONVROT_PROBE_FP6: 2 * 32 * 32 * 64, CONVROT_PROBE_INT8: 2 * 32 * 32 * 32}


def convrot_matrix_core_probe(kind: int, iterations: int, out=None, stream=None):
    """Enqueue the MFMA-only rate loop; returns (MFMA instructions it runs, out).
    The caller times it on the stream."""
    import torch
    if out is None:
        nbytes = _SZ(0)
        _call("convrot_matrix_core_probe_bytes", ctypes.byref(nbytes))
        out = torch.empty(nbytes.value // 4, dtype=torch.float32, device="cuda")
    count = _I64(0)
    _call("convrot_matrix_core_probe", kind, iterations, _dev(out, torch.float32, "out"), out.numel() * 4,
          ctypes.byref(count), _stream(stream))
    return count.value, out


def workspace_status(workspace) -> int:
    """The workspace's status word after a completed call (0, or CONVROT_STATUS_SPLIT_TIMEOUT)."""
    import torch
    return int(workspace[WORKSPACE_STATUS_OFFSET:WORKSPACE_STATUS_OFFSET + 4].view(torch.int32).item())


# --------------------------------------------------------------------------
# host layout tools (numpy in, numpy out)
# --------------------------------------------------------------------------

def _np(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _hp(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def convrot_host_pack_nk(codes) -> np.ndarray:
    q = _np(codes, np.int8)
    N, K = q.shape
    out = np.empty((N, K // 2), np.uint8)
    _call("convrot_host_pack_nk", _hp(q), N, K, _hp(out))
    return out


def convrot_host_unpack_nk(nk, K: int) -> np.ndarray:
    p = _np(nk, np.uint8)
    N = p.shape[0]
    out = np.empty((N, K), np.int8)
    _call("convrot_host_unpack_nk", _hp(p), N, K, _hp(out))
    return out


def convrot_host_nk_to_kn(nk, N: int, K: int) -> np.ndarray:
    p = _np(nk, np.uint8)
    out = np.empty((K, N // 2), np.uint8)
    _call("convrot_host_nk_to_kn", _hp(p), N, K, _hp(out))
    return out


def convrot_host_kn_to_nk(kn, N: int, K: int) -> np.ndarray:
    p = _np(kn, np.uint8)
    out = np.empty((N, K // 2), np.uint8)
    _call("convrot_host_kn_to_nk", _hp(p), N, K, _hp(out))
    return out


def convrot_host_nk_to_image(nk, N: int, K: int) -> np.ndarray:
    p = _np(nk, np.uint8)
    out = np.empty(convrot_weight_image_bytes(N, K, 64), np.uint8)
    _call("convrot_host_nk_to_image", _hp(p), N, K, _hp(out))
    return out


def convrot_host_image_to_nk(image, N: int, K: int) -> np.ndarray:
    p = _np(image, np.uint8)
    out = np.empty((N, K // 2), np.uint8)
    _call("convrot_host_image_to_nk", _hp(p), N, K, _hp(out))
    return out


def convrot_host_image_fp6_to_nk(image, N: int, K: int) -> np.ndarray:
    """The FP6 copy of the codes in a weight image, as N x packed-K."""
    p = _np(image, np.uint8)
    out = np.empty((N, K // 2), np.uint8)
    _call("convrot_host_image_fp6_to_nk", _hp(p), N, K, _hp(out))
    return out


def convrot_host_workspace_fp6_codes(workspace, M: int, K: int) -> np.ndarray:
    """The FP6 activation codes of a workspace (M > 32), as int8 [M, K]."""
    ws = workspace.cpu().numpy() if hasattr(workspace, "cpu") else np.asarray(workspace)
    p = _np(ws, np.uint8)
    out = np.empty((M, K), np.int8)
    _call("convrot_host_workspace_fp6_codes", _hp(p), M, K, _hp(out))
    return out


# Offset of the activation-code image inside a workspace
# (CONVROT_WORKSPACE_IMAGE_OFFSET in include/convrot.h).
WORKSPACE_IMAGE_OFFSET = 4096


def workspace_act_codes(workspace, M: int, K: int) -> np.ndarray:
    """Activation codes int8 [M, K] decoded from a workspace (tensor or array); K is
    the code width (the rotated width of the prepared rows)."""
    ws = workspace.cpu().numpy() if hasattr(workspace, "cpu") else np.asarray(workspace)
    return convrot_host_act_image_to_codes(ws[WORKSPACE_IMAGE_OFFSET:], M, K)


def convrot_host_act_image_to_codes(image, M: int, K: int) -> np.ndarray:
    p = _np(image, np.uint8)
    out = np.empty((M, K), np.int8)
    _call("convrot_host_act_image_to_codes", _hp(p), M, K, _hp(out))
    return out


# --------------------------------------------------------------------------
# W4A16 variant (M <= 32)
# --------------------------------------------------------------------------

def convrot_w4a16_workspace_bytes(M: int, K: int, g: int) -> int:
    out = ctypes.c_size_t()
    _call("convrot_w4a16_workspace_bytes", M, K, g, ctypes.byref(out))
    return out.value


def convrot_validate_linear_w4a16(X_ptr, M, K, image_ptr, sw_ptr, bias_ptr, N, g, Y_ptr, ws_ptr, ws_bytes) -> int:
    """Raw pointer values (ints); returns the status code."""
    return load().convrot_validate_linear_w4a16(X_ptr, M, K, image_ptr, sw_ptr, bias_ptr, N, g, Y_ptr, ws_ptr,
                                                ws_bytes)


def convrot_linear_w4a16(X, image, sw, bias, N: int, g: int, Y=None, workspace=None, stream=None):
    """Y = X W^T + bias with INT4 weights and bf16 rotated activations (M <= 32).
    The workspace receives the bf16 rotated rows [M, K]."""
    import torch
    M, K = X.shape
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    if workspace is None:
        workspace = torch.empty(max(convrot_w4a16_workspace_bytes(M, K, g), 1), dtype=torch.uint8, device=X.device)
    bias_p = None if bias is None else _dev(bias, torch.bfloat16, "bias")
    _call("convrot_linear_w4a16", _dev(X, torch.bfloat16, "X"), M, K, _dev(image, torch.uint8, "image"),
          _dev(sw, torch.float32, "sw"), bias_p, N, g, _dev(Y, torch.bfloat16, "Y"),
          _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream))
    return Y
