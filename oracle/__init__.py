"""CPU oracle for the ConvRot W4A4 rotated linear.

TEST INFRASTRUCTURE ONLY.  The test suite, the package's smoke check and the
benchmark's CPU-baseline leg are the only callers.  The product path (the HIP
library and its binding) never imports this package, and this package never
imports the product: the two share nothing but the seeded input generators,
which hold none of the method's arithmetic.

The arithmetic lives in ``convrot_oracle.c`` (plain loops, binary64 rotation,
binary32 quantization, int64 dot products).  This module only marshals numpy
arrays through ctypes; see the C file's header for the definition each
function follows and the pages' sections it cites.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "convrot_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc: -O2, no floating-point contraction."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread",
           "-std=c11", "-Wall", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def default_threads() -> int:
    env = os.environ.get("CONVROT_ORACLE_THREADS")
    if env:
        return max(1, int(env))
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_f32.restype = ctypes.c_float
        lib.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
        lib.oracle_f32_to_bf16_array.argtypes = [P, I64, P]
        lib.oracle_f32_to_bf16_array.restype = None
        lib.oracle_sylvester.argtypes = [I, P]
        lib.oracle_sylvester.restype = I
        lib.oracle_regular_hadamard.argtypes = [I, P]
        lib.oracle_regular_hadamard.restype = I
        lib.oracle_rotate_rows.argtypes = [P, I64, I64, I, P, I]
        lib.oracle_rotate_rows.restype = I
        lib.oracle_quantize_rows.argtypes = [P, I64, I64, P, P, I]
        lib.oracle_quantize_rows.restype = I
        lib.oracle_prepare_rows.argtypes = [P, I64, I64, I, P, P, P, I]
        lib.oracle_prepare_rows.restype = I
        for name in ("oracle_pack_nk", "oracle_nk_to_kn", "oracle_kn_to_nk"):
            getattr(lib, name).argtypes = [P, I64, I64, P]
            getattr(lib, name).restype = I
        lib.oracle_unpack_nk.argtypes = [P, I64, I64, P]
        lib.oracle_unpack_nk.restype = I
        lib.oracle_gemm_i32.argtypes = [P, P, I64, I64, I64, P, I]
        lib.oracle_gemm_i32.restype = I
        lib.oracle_epilogue.argtypes = [P, P, P, P, I64, I64, P]
        lib.oracle_epilogue.restype = None
        lib.oracle_epilogue_f32.argtypes = [P, P, P, P, I64, I64, P, P]
        lib.oracle_epilogue_f32.restype = None
        lib.oracle_linear.argtypes = [P, I64, I64, P, P, P, I64, I, P, P, P, P, I]
        lib.oracle_linear.restype = I
        lib.oracle_linear_w4a16.argtypes = [P, I64, I64, P, P, P, I64, I, P, P, P, I]
        lib.oracle_linear_w4a16.restype = I
        _lib = lib
        return lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with status {rc}")


# --------------------------------------------------------------------------
# bf16 conversions
# --------------------------------------------------------------------------

def bf16_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 values (exact widening)."""
    b = _c(bits, np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(values) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even."""
    v = _c(values, np.float32)
    out = np.empty(v.shape, dtype=np.uint16)
    _load().oracle_f32_to_bf16_array(_ptr(v), v.size, _ptr(out))
    return out


# --------------------------------------------------------------------------
# the method's steps
# --------------------------------------------------------------------------

# Group-size flag (OR'd into g): rotate with the regular Hadamard matrix.
REGULAR = 0x10000


def rotated_width(K: int, g: int) -> int:
    """Rows are zero-padded to a whole number of groups: K rounded up to g."""
    gs = g & ~REGULAR
    return -(-K // gs) * gs


def sylvester(g: int) -> np.ndarray:
    """Integer Sylvester Hadamard matrix H_g (entries +-1), natural order."""
    H = np.empty((g, g), dtype=np.int8)
    _check(_load().oracle_sylvester(int(g), _ptr(H)), "sylvester")
    return H


def regular_hadamard(g: int) -> np.ndarray:
    """Integer regular Hadamard matrix (J_4 - 2 I_4)^(x k) of order g = 4^k."""
    H = np.empty((g, g), dtype=np.int8)
    _check(_load().oracle_regular_hadamard(int(g), _ptr(H)), "regular_hadamard")
    return H


def rotate_rows(x_bf16, g: int, threads: int | None = None) -> np.ndarray:
    """r = x (I_G (x) H_g) / sqrt(g), each group in binary64, rounded once to
    binary32; H is Sylvester, or regular when g carries REGULAR."""
    x = _c(x_bf16, np.uint16)
    rows, K = x.shape
    r = np.empty((rows, rotated_width(K, g)), dtype=np.float32)
    _check(_load().oracle_rotate_rows(_ptr(x), rows, K, int(g), _ptr(r), threads or default_threads()),
           "rotate_rows")
    return r


def quantize_rows(r32, threads: int | None = None):
    """Rowwise absmax/7 scale and codes clamp(rint(r/s), -7, 7).  Returns (codes int8, scales f32)."""
    r = _c(r32, np.float32)
    rows, K = r.shape
    q = np.empty((rows, K), dtype=np.int8)
    s = np.empty((rows,), dtype=np.float32)
    _check(_load().oracle_quantize_rows(_ptr(r), rows, K, _ptr(q), _ptr(s), threads or default_threads()),
           "quantize_rows")
    return q, s


def prepare_rows(x_bf16, g: int, threads: int | None = None, want_rotated: bool = False):
    """Rotate + quantize rows of a bf16 matrix (activations X or weights W).

    Returns (codes int8 [rows, K], scales f32 [rows]) and, if asked, the
    binary32 rotated values."""
    x = _c(x_bf16, np.uint16)
    rows, K = x.shape
    Kr = rotated_width(K, g)
    q = np.empty((rows, Kr), dtype=np.int8)
    s = np.empty((rows,), dtype=np.float32)
    r = np.empty((rows, Kr), dtype=np.float32) if want_rotated else None
    _check(_load().oracle_prepare_rows(_ptr(x), rows, K, int(g), _ptr(q), _ptr(s), _ptr(r),
                                       threads or default_threads()), "prepare_rows")
    return (q, s, r) if want_rotated else (q, s)


def pack_nk(codes) -> np.ndarray:
    """int8 codes [N, K] -> uint8 N x packed-K [N, K/2] (low nibble = even k)."""
    q = _c(codes, np.int8)
    N, K = q.shape
    p = np.empty((N, K // 2), dtype=np.uint8)
    _check(_load().oracle_pack_nk(_ptr(q), N, K, _ptr(p)), "pack_nk")
    return p


def unpack_nk(packed, K: int) -> np.ndarray:
    p = _c(packed, np.uint8)
    N = p.shape[0]
    q = np.empty((N, K), dtype=np.int8)
    _check(_load().oracle_unpack_nk(_ptr(p), N, K, _ptr(q)), "unpack_nk")
    return q


def nk_to_kn(packed_nk, N: int, K: int) -> np.ndarray:
    """N x packed-K [N, K/2] -> K x packed-N [K, N/2] (low nibble = even n)."""
    p = _c(packed_nk, np.uint8)
    out = np.empty((K, N // 2), dtype=np.uint8)
    _check(_load().oracle_nk_to_kn(_ptr(p), N, K, _ptr(out)), "nk_to_kn")
    return out


def kn_to_nk(packed_kn, N: int, K: int) -> np.ndarray:
    p = _c(packed_kn, np.uint8)
    out = np.empty((N, K // 2), dtype=np.uint8)
    _check(_load().oracle_kn_to_nk(_ptr(p), N, K, _ptr(out)), "kn_to_nk")
    return out


def gemm_i32(qx, qw, threads: int | None = None) -> np.ndarray:
    """acc[m, n] = sum_k qx[m, k] * qw[n, k], summed in int64; raises if a sum leaves int32."""
    a = _c(qx, np.int8)
    b = _c(qw, np.int8)
    M, K = a.shape
    N = b.shape[0]
    assert b.shape[1] == K
    acc = np.empty((M, N), dtype=np.int32)
    rc = _load().oracle_gemm_i32(_ptr(a), _ptr(b), M, N, K, _ptr(acc), threads or default_threads())
    if rc == 1:
        raise OverflowError("integer dot product does not fit int32")
    _check(rc, "gemm_i32")
    return acc


def epilogue(acc, sx, sw, bias_bf16=None, want_f32: bool = False):
    """Y = bf16(fmaf(float(acc) * sx[m], sw[n], bias[n])), returned as bf16 bits
    (and, if asked, the binary32 values before the bf16 rounding)."""
    a = _c(acc, np.int32)
    M, N = a.shape
    sxa = _c(sx, np.float32)
    swa = _c(sw, np.float32)
    b = None if bias_bf16 is None else _c(bias_bf16, np.uint16)
    y = np.empty((M, N), dtype=np.uint16)
    yf = np.empty((M, N), dtype=np.float32) if want_f32 else None
    _load().oracle_epilogue_f32(_ptr(a), _ptr(sxa), _ptr(swa), _ptr(b), M, N, _ptr(y), _ptr(yf))
    return (y, yf) if want_f32 else y


def prepare_weight(w_bf16, g: int, threads: int | None = None):
    """Offline weight preparation: rotate + rowwise-quantize.  Returns (codes [N, K], sw [N])."""
    return prepare_rows(w_bf16, g, threads)


def linear(x_bf16, qw_codes, sw, bias_bf16, g: int, threads: int | None = None, want_parts: bool = False):
    """The whole linear: prepare X rows, integer products against the weight
    codes, scale + bias epilogue.  Returns Y as bf16 bits [M, N] (and, if
    asked, a dict with the activation codes, scales and int32 sums)."""
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    qw = _c(qw_codes, np.int8)
    N = qw.shape[0]
    if qw.shape[1] != rotated_width(K, g):
        raise ValueError("weight codes must be K rounded up to g wide")
    swa = _c(sw, np.float32)
    b = None if bias_bf16 is None else _c(bias_bf16, np.uint16)
    y = np.empty((M, N), dtype=np.uint16)
    qx = np.empty((M, rotated_width(K, g)), dtype=np.int8) if want_parts else None
    sx = np.empty((M,), dtype=np.float32) if want_parts else None
    acc = np.empty((M, N), dtype=np.int32) if want_parts else None
    rc = _load().oracle_linear(_ptr(x), M, K, _ptr(qw), _ptr(swa), _ptr(b), N, int(g), _ptr(y), _ptr(qx),
                               _ptr(sx), _ptr(acc), threads or default_threads())
    if rc == 1:
        raise OverflowError("integer dot product does not fit int32")
    _check(rc, "linear")
    if want_parts:
        return y, {"qx": qx, "sx": sx, "acc": acc}
    return y


def linear_w4a16(x_bf16, qw_codes, sw, bias_bf16, g: int, threads: int | None = None, want_rotated: bool = False,
                 want_f32: bool = False):
    """W4A16: rotated activation rows rounded to bf16, times the INT4 weight
    codes (exact products, binary64 sum), y = fmaf(fl32(sum), sw, bias) to bf16.
    Returns Y as bf16 bits [M, N] (and, if asked, the bf16 rotated X and the
    binary32 outputs before the bf16 rounding, in that order)."""
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    qw = _c(qw_codes, np.int8)
    N = qw.shape[0]
    if qw.shape[1] != rotated_width(K, g):
        raise ValueError("weight codes must be K rounded up to g wide")
    swa = _c(sw, np.float32)
    b = None if bias_bf16 is None else _c(bias_bf16, np.uint16)
    y = np.empty((M, N), dtype=np.uint16)
    xr = np.empty((M, rotated_width(K, g)), dtype=np.uint16) if want_rotated else None
    yf = np.empty((M, N), dtype=np.float32) if want_f32 else None
    _check(_load().oracle_linear_w4a16(_ptr(x), M, K, _ptr(qw), _ptr(swa), _ptr(b), N, int(g), _ptr(y), _ptr(xr),
                                       _ptr(yf), threads or default_threads()), "linear_w4a16")
    out = (y,) + ((xr,) if want_rotated else ()) + ((yf,) if want_f32 else ())
    return out if len(out) > 1 else y
