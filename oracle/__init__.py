"""Oracle for the W1.58A8 ternary matrix product (Python side).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It wraps the plain C oracle in
``oracle.c`` (scalar loops, no HIP) with numpy arrays and shares no code with
the GPU library.  The functions follow the pages cited in ``oracle.h``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
          "-shared", "-pthread"]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no HIP involved)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        i64, i32, p = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.oracle_ternarize_absmean.argtypes = [p, i64, i64, p, p]
        L.oracle_ternarize_absmean.restype = i32
        L.oracle_pack_i2s.argtypes = [p, i64, i64, p]
        L.oracle_pack_i2s.restype = i64
        L.oracle_unpack_i2s.argtypes = [p, i64, i64, p]
        L.oracle_unpack_i2s.restype = i64
        L.oracle_b3_packed_bytes.argtypes = [i64, i64]
        L.oracle_b3_packed_bytes.restype = i64
        L.oracle_pack_b3.argtypes = [p, i64, i64, p]
        L.oracle_pack_b3.restype = i64
        L.oracle_unpack_b3.argtypes = [p, i64, i64, p]
        L.oracle_unpack_b3.restype = i64
        L.oracle_rmsnorm.argtypes = [p, p, i64, i64, ctypes.c_float, p, p]
        L.oracle_rmsnorm.restype = i32
        L.oracle_quant_act.argtypes = [p, i64, i64, p, p]
        L.oracle_quant_act.restype = i32
        L.oracle_gemm.argtypes = [p, ctypes.c_float, i64, i64, i64, p, p, i64,
                                  i64, p, p, i32]
        L.oracle_gemm.restype = i32
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def ternarize_absmean(w):
    """O1: fp32 [n, k] -> (int8 trits [n, k], fp32 scale)."""
    w = _c(w, np.float32)
    n, k = w.shape
    t = np.empty((n, k), np.int8)
    s = np.zeros(1, np.float32)
    lib().oracle_ternarize_absmean(_ptr(w), n, k, _ptr(t), _ptr(s))
    return t, np.float32(s[0])


def packed_bytes(n: int, k: int) -> int:
    """Size of the O2 layout: rows padded to a multiple of 64, 2 bits each."""
    return (n + 63) // 64 * 64 * k // 4


def pack_i2s(t):
    """O2: int8 trits [n, k] -> (uint8 packed, flat, invalid count)."""
    t = _c(t, np.int8)
    n, k = t.shape
    if k % 64:
        raise ValueError("k must be a multiple of 64")
    out = np.empty(packed_bytes(n, k), np.uint8)
    bad = lib().oracle_pack_i2s(_ptr(t), n, k, _ptr(out))
    return out, int(bad)


def unpack_i2s(packed, n: int, k: int):
    """O2 inverse: packed bytes -> (int8 trits [n, k], invalid count)."""
    packed = _c(packed, np.uint8).ravel()
    if packed.size != packed_bytes(n, k):
        raise ValueError("packed size does not match n, k")
    t = np.empty((n, k), np.int8)
    bad = lib().oracle_unpack_i2s(_ptr(packed), n, k, _ptr(t))
    return t, int(bad)


def b3_packed_bytes(n: int, k: int) -> int:
    """Size of the base-3 layout (five trits per byte; rows padded to 64,
    inputs to 80)."""
    return int(lib().oracle_b3_packed_bytes(n, k))


def pack_b3(t):
    """Five trits per byte: int8 trits [n, k] -> (uint8 packed, invalid
    count)."""
    t = _c(t, np.int8)
    n, k = t.shape
    out = np.empty(b3_packed_bytes(n, k), np.uint8)
    bad = lib().oracle_pack_b3(_ptr(t), n, k, _ptr(out))
    return out, int(bad)


def unpack_b3(packed, n: int, k: int):
    """Inverse of pack_b3 -> (int8 trits [n, k], count of bytes the packer
    cannot have written)."""
    packed = _c(packed, np.uint8).ravel()
    if packed.size != b3_packed_bytes(n, k):
        raise ValueError("packed size does not match n, k")
    t = np.empty((n, k), np.int8)
    bad = lib().oracle_unpack_b3(_ptr(packed), n, k, _ptr(t))
    return t, int(bad)


def quant_act(x):
    """O3: fp32 [m, k] -> (int8 q [m, k], fp32 s_a [m])."""
    x = _c(x, np.float32)
    if x.ndim == 1:
        x = x[None, :]
    m, k = x.shape
    q = np.empty((m, k), np.int8)
    s = np.empty(m, np.float32)
    lib().oracle_quant_act(_ptr(x), m, k, _ptr(q), _ptr(s))
    return q, s


def rmsnorm(x, g, eps: float):
    """RMSNorm of fp32 rows x [m, k] with gain g [k] -> (fp32 h [m, k],
    float64 r64 [m], the scale before its rounding to fp32)."""
    x = _c(x, np.float32)
    if x.ndim == 1:
        x = x[None, :]
    g = _c(g, np.float32).ravel()
    m, k = x.shape
    if g.size != k:
        raise ValueError("g must have k elements")
    h = np.empty((m, k), np.float32)
    r64 = np.empty(m, np.float64)
    lib().oracle_rmsnorm(_ptr(x), _ptr(g), m, k, float(np.float32(eps)),
                         _ptr(h), _ptr(r64))
    return h, r64


def rmsnorm_quant(x, g, eps: float):
    """RMSNorm then O3: fp32 [m, k] -> (int8 q, fp32 s_a, fp32 h, r64)."""
    h, r64 = rmsnorm(x, g, eps)
    q, s_a = quant_act(h)
    return q, s_a, h, r64


def gemm(packed, s_w, n: int, k: int, q, s_a, nthreads: int = 1, rows=None):
    """O4 + O5: (int32 acc [m, r1-r0], float64 y [m, r1-r0]).

    ``rows`` = (r0, r1) restricts the product to output rows r0..r1-1 (used to
    compute samples at full sizes); the default is every row."""
    packed = _c(packed, np.uint8).ravel()
    q = _c(q, np.int8)
    if q.ndim == 1:
        q = q[None, :]
    s_a = _c(np.atleast_1d(s_a), np.float32)
    m = q.shape[0]
    r0, r1 = (0, n) if rows is None else rows
    if (packed.size != packed_bytes(n, k) or q.shape[1] != k
            or s_a.shape[0] != m):
        raise ValueError("shape mismatch")
    acc = np.empty((m, r1 - r0), np.int32)
    y = np.empty((m, r1 - r0), np.float64)
    rc = lib().oracle_gemm(_ptr(packed), float(np.float32(s_w)), n, k, m,
                           _ptr(q), _ptr(s_a), r0, r1, _ptr(acc), _ptr(y),
                           int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_gemm failed with {rc}")
    return acc, y


def rescale_f32(acc, s_w, s_a):
    """O5 in the method's own precision: y = ((float)acc * s_w) * s_a, two
    fp32 multiplies left to right (config C1 writes the rescale in that
    order; bitnet.cpp CPU tutorial §1.1 for the integer product it scales).
    The fp64 ``y`` of ``gemm`` is the exact value; this is the fp32 result a
    consumer of the output sees, e.g. the next quantization of a chained
    decode."""
    acc = np.asarray(acc)
    a32 = acc.astype(np.float32)
    if not np.array_equal(a32.astype(np.int64), acc.astype(np.int64)):
        raise ValueError("accumulator not exact in fp32")
    s_a = np.asarray(s_a, np.float32).reshape(-1, 1)
    return (a32 * np.float32(s_w)).astype(np.float32) * s_a
