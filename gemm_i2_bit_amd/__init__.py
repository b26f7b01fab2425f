"""Python binding of libbt, the MI355X (gfx950) ternary W1.58A8 GEMV/GEMM
library.  Argument marshalling only: every step of the product runs in the
library's HIP kernels.  PyTorch supplies device memory and streams.

Functions carry the C ABI's names (see include/bt.h for the contract):
bt_pack_i2s, bt_quant_act, bt_quant_act_many, bt_gemv, bt_gemm,
bt_grouped_plan (and bt_grouped_plan_xcd through its xcd_shares argument),
bt_grouped_plan_f32, bt_gemm_grouped, bt_packed_bytes,
bt_status_str, and the measurement helpers bt_read_probe and bt_mix_probe.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbt.so")

BT_OK, BT_E_NULL, BT_E_SHAPE, BT_E_ALIGN, BT_E_ARG, BT_E_HIP, BT_E_ARCH = (
    0, -1, -2, -3, -4, -5, -6)

BT_MAX_M = 1 << 24
BT_MAX_QUANT_JOBS = 16
BT_FUSED_MAX_MK = 16384
BT_STATIC_SCRATCH_BYTES = 32 << 20
BT_CHAIN_STATUS_OFFSET = 4356

_lib = None


class BtError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {bt_status_str(status)} (status {status})")


class bt_problem(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("x_q", ctypes.c_void_p),
                ("s_a", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("acc", ctypes.c_void_p), ("s_w", ctypes.c_float),
                ("n", ctypes.c_int32), ("k", ctypes.c_int32),
                ("m", ctypes.c_int32)]


class bt_problem_f32(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("x", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("acc", ctypes.c_void_p),
                ("s_w", ctypes.c_float), ("n", ctypes.c_int32),
                ("k", ctypes.c_int32), ("m", ctypes.c_int32)]


class bt_problem_norm(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("x", ctypes.c_void_p),
                ("g", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("acc", ctypes.c_void_p), ("s_w", ctypes.c_float),
                ("eps", ctypes.c_float), ("n", ctypes.c_int32),
                ("k", ctypes.c_int32), ("m", ctypes.c_int32)]


class bt_chain_phase(ctypes.Structure):
    _fields_ = [("plan_dev", ctypes.c_void_p), ("plan_host", ctypes.c_void_p)]


class bt_quant_job(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("x_q", ctypes.c_void_p),
                ("s_a", ctypes.c_void_p), ("m", ctypes.c_int64),
                ("k", ctypes.c_int64)]


def lib() -> ctypes.CDLL:
    """Load libbt.so; fails loudly when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python gemm_i2_bit_amd/build.py` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        p, i32, i64, f32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                            ctypes.c_float)
        L.bt_status_str.argtypes = [i32]
        L.bt_status_str.restype = ctypes.c_char_p
        L.bt_packed_bytes.argtypes = [i64, i64]
        L.bt_packed_bytes.restype = i64
        L.bt_pack_i2s.argtypes = [p, i64, i64, p, p, p]
        L.bt_pack_i2s.restype = i32
        L.bt_quant_act.argtypes = [p, i64, i64, p, p, p]
        L.bt_quant_act.restype = i32
        L.bt_quant_act_many.argtypes = [p, i32, p]
        L.bt_quant_act_many.restype = i32
        L.bt_gemv.argtypes = [p, f32, i64, i64, p, p, p, p, p]
        L.bt_gemv.restype = i32
        L.bt_gemv_lut.argtypes = [p, f32, i64, i64, p, p, p, p, p]
        L.bt_gemv_lut.restype = i32
        L.bt_gemm.argtypes = [p, f32, i64, i64, i64, p, p, p, p, p]
        L.bt_gemm.restype = i32
        L.bt_grouped_plan_bytes.argtypes = [p, i32]
        L.bt_grouped_plan_bytes.restype = i64
        L.bt_grouped_plan.argtypes = [p, i32, p, i64]
        L.bt_grouped_plan.restype = i32
        L.bt_grouped_plan_xcd.argtypes = [p, i32, p, i32, p, i64]
        L.bt_grouped_plan_xcd.restype = i32
        L.bt_grouped_plan_f32_bytes.argtypes = [p, i32]
        L.bt_grouped_plan_f32_bytes.restype = i64
        L.bt_grouped_plan_f32.argtypes = [p, i32, p, i64]
        L.bt_grouped_plan_f32.restype = i32
        L.bt_gemm_grouped.argtypes = [p, p, p]
        L.bt_gemm_grouped.restype = i32
        L.bt_b3_packed_bytes.argtypes = [i64, i64]
        L.bt_b3_packed_bytes.restype = i64
        L.bt_pack_b3.argtypes = [p, i64, i64, p, p, p]
        L.bt_pack_b3.restype = i32
        L.bt_gemv_b3.argtypes = [p, f32, i64, i64, p, p, p, p, p]
        L.bt_gemv_b3.restype = i32
        L.bt_rmsnorm_quant.argtypes = [p, p, i64, i64, f32, p, p, p, p]
        L.bt_rmsnorm_quant.restype = i32
        L.bt_grouped_plan_norm_bytes.argtypes = [p, i32]
        L.bt_grouped_plan_norm_bytes.restype = i64
        L.bt_grouped_plan_norm.argtypes = [p, i32, p, i64]
        L.bt_grouped_plan_norm.restype = i32
        L.bt_chain_plan_bytes.argtypes = [i32]
        L.bt_chain_plan_bytes.restype = i64
        L.bt_chain_plan.argtypes = [p, i32, p, i64]
        L.bt_chain_plan.restype = i32
        L.bt_gemm_chain.argtypes = [p, p, p]
        L.bt_gemm_chain.restype = i32
        L.bt_gemm_grouped_static.argtypes = [p, p, p]
        L.bt_gemm_grouped_static.restype = i32
        L.bt_read_probe.argtypes = [p, i64, p, i64, i32, i32, p]
        L.bt_read_probe.restype = i32
        L.bt_mix_probe.argtypes = [p, i64, p, i64, i32, p, i64, i32, i32, p]
        L.bt_mix_probe.restype = i32
        _lib = L
    return _lib


def bt_status_str(status: int) -> str:
    return lib().bt_status_str(int(status)).decode()


def _check(status: int, what: str):
    if status != BT_OK:
        raise BtError(status, what)


def _torch():
    import torch
    return torch


def _dev(t, dtype, name):
    """Pointer of a contiguous GPU tensor of the given dtype (None -> NULL)."""
    if t is None:
        return None
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def bt_packed_bytes(n: int, k: int) -> int:
    r = lib().bt_packed_bytes(n, k)
    if r < 0:
        raise BtError(r, "bt_packed_bytes")
    return r


def bt_pack_i2s(t, packed=None, n_invalid=None, stream=None):
    """int8 trits [n, k] (GPU) -> packed uint8 (GPU, bt_packed_bytes)."""
    torch = _torch()
    n, k = t.shape
    if packed is None:
        packed = torch.empty(bt_packed_bytes(n, k), dtype=torch.uint8,
                             device=t.device)
    if packed.numel() != bt_packed_bytes(n, k):
        raise ValueError("packed has the wrong size")
    _check(lib().bt_pack_i2s(_dev(t, torch.int8, "t"), n, k,
                             _dev(packed, torch.uint8, "packed"),
                             _dev(n_invalid, torch.int32, "n_invalid"),
                             _stream(stream)), "bt_pack_i2s")
    return packed


def bt_quant_act(x, x_q=None, s_a=None, stream=None):
    """fp32 [m, k] (GPU) -> (int8 x_q [m, k], fp32 s_a [m])."""
    torch = _torch()
    if x.dim() == 1:
        x = x.unsqueeze(0)
    m, k = x.shape
    if x_q is None:
        x_q = torch.empty((m, k), dtype=torch.int8, device=x.device)
    if s_a is None:
        s_a = torch.empty(m, dtype=torch.float32, device=x.device)
    if x_q.numel() != m * k or s_a.numel() != m:
        raise ValueError("x_q or s_a has the wrong size")
    _check(lib().bt_quant_act(_dev(x, torch.float32, "x"), m, k,
                              _dev(x_q, torch.int8, "x_q"),
                              _dev(s_a, torch.float32, "s_a"),
                              _stream(stream)), "bt_quant_act")
    return x_q, s_a


def bt_rmsnorm_quant(x, g, eps: float, x_q=None, s_a=None, h=None,
                     want_h: bool = False, stream=None):
    """RMSNorm (gain g [k], eps) then absmax quantization of fp32 [m, k]
    (GPU) -> (int8 x_q, fp32 s_a, fp32 h or None)."""
    torch = _torch()
    if x.dim() == 1:
        x = x.unsqueeze(0)
    m, k = x.shape
    if x_q is None:
        x_q = torch.empty((m, k), dtype=torch.int8, device=x.device)
    if s_a is None:
        s_a = torch.empty(m, dtype=torch.float32, device=x.device)
    if h is None and want_h:
        h = torch.empty((m, k), dtype=torch.float32, device=x.device)
    if (x_q.numel() != m * k or s_a.numel() != m or g.numel() != k
            or (h is not None and h.numel() != m * k)):
        raise ValueError("x_q, s_a, g or h has the wrong size")
    _check(lib().bt_rmsnorm_quant(_dev(x, torch.float32, "x"),
                                  _dev(g, torch.float32, "g"), m, k,
                                  float(eps), _dev(x_q, torch.int8, "x_q"),
                                  _dev(s_a, torch.float32, "s_a"),
                                  _dev(h, torch.float32, "h"),
                                  _stream(stream)), "bt_rmsnorm_quant")
    return x_q, s_a, h


def bt_quant_act_many(xs, x_qs=None, s_as=None, stream=None):
    """Several fp32 [m_j, k_j] (GPU) in one launch -> lists of int8 x_q and
    fp32 s_a, each as bt_quant_act would give."""
    torch = _torch()
    xs = [x.unsqueeze(0) if x.dim() == 1 else x for x in xs]
    if x_qs is None:
        x_qs = [torch.empty(x.shape, dtype=torch.int8, device=x.device)
                for x in xs]
    if s_as is None:
        s_as = [torch.empty(x.shape[0], dtype=torch.float32, device=x.device)
                for x in xs]
    if not (len(xs) == len(x_qs) == len(s_as)):
        raise ValueError("xs, x_qs and s_as differ in length")
    arr = (bt_quant_job * max(len(xs), 1))()
    for j, (x, q, s) in enumerate(zip(xs, x_qs, s_as)):
        m, k = x.shape
        if q.numel() != m * k or s.numel() != m:
            raise ValueError(f"job {j}: x_q or s_a has the wrong size")
        arr[j] = bt_quant_job(_dev(x, torch.float32, "x"),
                              _dev(q, torch.int8, "x_q"),
                              _dev(s, torch.float32, "s_a"), m, k)
    _check(lib().bt_quant_act_many(arr, len(xs), _stream(stream)),
           "bt_quant_act_many")
    return x_qs, s_as


def _outputs(m, n, device, y, acc, want_acc):
    torch = _torch()
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=device)
    if acc is None and want_acc:
        acc = torch.empty((m, n), dtype=torch.int32, device=device)
    if y.numel() != m * n or (acc is not None and acc.numel() != m * n):
        raise ValueError("y or acc has the wrong size")
    return y, acc


def bt_gemm(packed, s_w, n: int, k: int, x_q, s_a, y=None, acc=None,
            want_acc: bool = False, stream=None):
    """y [m, n] = (trits . x_q) * s_w * s_a; returns (y, acc or None)."""
    torch = _torch()
    m = x_q.shape[0] if x_q.dim() == 2 else 1
    if x_q.numel() != m * k or s_a.numel() != m:
        raise ValueError("x_q or s_a has the wrong size")
    if packed.numel() != bt_packed_bytes(n, k):
        raise ValueError("packed has the wrong size")
    y, acc = _outputs(m, n, x_q.device, y, acc, want_acc)
    _check(lib().bt_gemm(_dev(packed, torch.uint8, "packed"), float(s_w), n,
                         k, m, _dev(x_q, torch.int8, "x_q"),
                         _dev(s_a, torch.float32, "s_a"),
                         _dev(y, torch.float32, "y"),
                         _dev(acc, torch.int32, "acc"), _stream(stream)),
           "bt_gemm")
    return y, acc


def bt_gemv(packed, s_w, n: int, k: int, x_q, s_a, y=None, acc=None,
            want_acc: bool = False, stream=None):
    """One token: x_q [k] or [1, k] -> y [1, n]."""
    torch = _torch()
    if x_q.numel() != k or s_a.numel() != 1:
        raise ValueError("x_q or s_a has the wrong size")
    if packed.numel() != bt_packed_bytes(n, k):
        raise ValueError("packed has the wrong size")
    y, acc = _outputs(1, n, x_q.device, y, acc, want_acc)
    _check(lib().bt_gemv(_dev(packed, torch.uint8, "packed"), float(s_w), n,
                         k, _dev(x_q, torch.int8, "x_q"),
                         _dev(s_a, torch.float32, "s_a"),
                         _dev(y, torch.float32, "y"),
                         _dev(acc, torch.int32, "acc"), _stream(stream)),
           "bt_gemv")
    return y, acc


def bt_gemv_lut(packed, s_w, n: int, k: int, x_q, s_a, y=None, acc=None,
                want_acc: bool = False, stream=None):
    """bt_gemv computed with lookup tables (for comparison)."""
    torch = _torch()
    if x_q.numel() != k or s_a.numel() != 1:
        raise ValueError("x_q or s_a has the wrong size")
    if packed.numel() != bt_packed_bytes(n, k):
        raise ValueError("packed has the wrong size")
    y, acc = _outputs(1, n, x_q.device, y, acc, want_acc)
    _check(lib().bt_gemv_lut(_dev(packed, torch.uint8, "packed"), float(s_w),
                             n, k, _dev(x_q, torch.int8, "x_q"),
                             _dev(s_a, torch.float32, "s_a"),
                             _dev(y, torch.float32, "y"),
                             _dev(acc, torch.int32, "acc"), _stream(stream)),
           "bt_gemv_lut")
    return y, acc


def bt_b3_packed_bytes(n: int, k: int) -> int:
    r = lib().bt_b3_packed_bytes(n, k)
    if r < 0:
        raise BtError(r, "bt_b3_packed_bytes")
    return r


def bt_pack_b3(t, packed=None, n_invalid=None, stream=None):
    """int8 trits [n, k] (GPU) -> uint8 packed five per byte (GPU,
    bt_b3_packed_bytes)."""
    torch = _torch()
    n, k = t.shape
    if packed is None:
        packed = torch.empty(bt_b3_packed_bytes(n, k), dtype=torch.uint8,
                             device=t.device)
    if packed.numel() != bt_b3_packed_bytes(n, k):
        raise ValueError("packed has the wrong size")
    _check(lib().bt_pack_b3(_dev(t, torch.int8, "t"), n, k,
                            _dev(packed, torch.uint8, "packed"),
                            _dev(n_invalid, torch.int32, "n_invalid"),
                            _stream(stream)), "bt_pack_b3")
    return packed


def bt_gemv_b3(packed, s_w, n: int, k: int, x_q, s_a, y=None, acc=None,
               want_acc: bool = False, stream=None):
    """bt_gemv over weights packed by bt_pack_b3."""
    torch = _torch()
    if x_q.numel() != k or s_a.numel() != 1:
        raise ValueError("x_q or s_a has the wrong size")
    if packed.numel() != bt_b3_packed_bytes(n, k):
        raise ValueError("packed has the wrong size")
    y, acc = _outputs(1, n, x_q.device, y, acc, want_acc)
    _check(lib().bt_gemv_b3(_dev(packed, torch.uint8, "packed"), float(s_w),
                            n, k, _dev(x_q, torch.int8, "x_q"),
                            _dev(s_a, torch.float32, "s_a"),
                            _dev(y, torch.float32, "y"),
                            _dev(acc, torch.int32, "acc"), _stream(stream)),
           "bt_gemv_b3")
    return y, acc


class GroupedPlan:
    """A grouped-product plan: the host image and its device copy.  Keeps
    references to every tensor the plan points at."""

    def __init__(self, host: np.ndarray, dev, tensors):
        self.host = host
        self.dev = dev
        self._tensors = tensors


def bt_grouped_plan(problems, device=None, xcd_shares=None) -> GroupedPlan:
    """problems: list of dicts with packed, s_w, n, k, x_q, s_a, y and
    optionally acc (GPU tensors; every problem has the same m).  xcd_shares:
    optional per-XCD shares in permille (bt_grouped_plan_xcd)."""
    torch = _torch()
    arr = (bt_problem * len(problems))()
    keep = []
    for i, p in enumerate(problems):
        m = p["x_q"].shape[0] if p["x_q"].dim() == 2 else 1
        if (p["x_q"].numel() != m * p["k"] or p["s_a"].numel() != m
                or p["y"].numel() != m * p["n"]
                or p["packed"].numel() != bt_packed_bytes(p["n"], p["k"])
                or (p.get("acc") is not None
                    and p["acc"].numel() != m * p["n"])):
            raise ValueError(f"problem {i} has inconsistent sizes")
        arr[i] = bt_problem(_dev(p["packed"], torch.uint8, "packed"),
                            _dev(p["x_q"], torch.int8, "x_q"),
                            _dev(p["s_a"], torch.float32, "s_a"),
                            _dev(p["y"], torch.float32, "y"),
                            _dev(p.get("acc"), torch.int32, "acc"),
                            float(p["s_w"]), p["n"], p["k"], m)
        keep.append(p)
    nbytes = lib().bt_grouped_plan_bytes(arr, len(problems))
    if nbytes < 0:
        raise BtError(nbytes, "bt_grouped_plan_bytes")
    host = np.zeros(nbytes, np.uint8)
    if xcd_shares is None:
        _check(lib().bt_grouped_plan(arr, len(problems), host.ctypes.data,
                                     nbytes), "bt_grouped_plan")
    else:
        sh = np.ascontiguousarray(xcd_shares, dtype=np.int32)
        _check(lib().bt_grouped_plan_xcd(arr, len(problems), sh.ctypes.data,
                                         sh.size, host.ctypes.data, nbytes),
               "bt_grouped_plan_xcd")
    if device is None:
        device = problems[0]["x_q"].device
    dev = torch.from_numpy(host).to(device)
    return GroupedPlan(host, dev, keep)


def bt_grouped_plan_f32(problems, device=None) -> GroupedPlan:
    """problems: list of dicts with packed, s_w, n, k, x (fp32 activations
    [m, k]), y and optionally acc (GPU tensors; one m <= 4 for all).  The
    launch quantizes x itself, as bt_quant_act would."""
    torch = _torch()
    arr = (bt_problem_f32 * len(problems))()
    keep = []
    for i, p in enumerate(problems):
        x = p["x"]
        m = x.shape[0] if x.dim() == 2 else 1
        if (x.numel() != m * p["k"] or p["y"].numel() != m * p["n"]
                or p["packed"].numel() != bt_packed_bytes(p["n"], p["k"])
                or (p.get("acc") is not None
                    and p["acc"].numel() != m * p["n"])):
            raise ValueError(f"problem {i} has inconsistent sizes")
        arr[i] = bt_problem_f32(_dev(p["packed"], torch.uint8, "packed"),
                                _dev(x, torch.float32, "x"),
                                _dev(p["y"], torch.float32, "y"),
                                _dev(p.get("acc"), torch.int32, "acc"),
                                float(p["s_w"]), p["n"], p["k"], m)
        keep.append(p)
    nbytes = lib().bt_grouped_plan_f32_bytes(arr, len(problems))
    if nbytes < 0:
        raise BtError(nbytes, "bt_grouped_plan_f32_bytes")
    host = np.zeros(nbytes, np.uint8)
    _check(lib().bt_grouped_plan_f32(arr, len(problems), host.ctypes.data,
                                     nbytes), "bt_grouped_plan_f32")
    if device is None:
        device = problems[0]["x"].device
    dev = torch.from_numpy(host).to(device)
    return GroupedPlan(host, dev, keep)


def bt_grouped_plan_norm(problems, device=None) -> GroupedPlan:
    """problems: list of dicts with packed, s_w, n, k, x (fp32 [m, k]), g
    (fp32 gain [k]), eps, y and optionally acc (GPU tensors; one m <= 4 for
    all).  The launch normalizes and quantizes x itself, as
    bt_rmsnorm_quant would."""
    torch = _torch()
    arr = (bt_problem_norm * len(problems))()
    keep = []
    for i, p in enumerate(problems):
        x = p["x"]
        m = x.shape[0] if x.dim() == 2 else 1
        if (x.numel() != m * p["k"] or p["y"].numel() != m * p["n"]
                or p["g"].numel() != p["k"]
                or p["packed"].numel() != bt_packed_bytes(p["n"], p["k"])
                or (p.get("acc") is not None
                    and p["acc"].numel() != m * p["n"])):
            raise ValueError(f"problem {i} has inconsistent sizes")
        arr[i] = bt_problem_norm(_dev(p["packed"], torch.uint8, "packed"),
                                 _dev(x, torch.float32, "x"),
                                 _dev(p["g"], torch.float32, "g"),
                                 _dev(p["y"], torch.float32, "y"),
                                 _dev(p.get("acc"), torch.int32, "acc"),
                                 float(p["s_w"]), float(p["eps"]), p["n"],
                                 p["k"], m)
        keep.append(p)
    nbytes = lib().bt_grouped_plan_norm_bytes(arr, len(problems))
    if nbytes < 0:
        raise BtError(nbytes, "bt_grouped_plan_norm_bytes")
    host = np.zeros(nbytes, np.uint8)
    _check(lib().bt_grouped_plan_norm(arr, len(problems), host.ctypes.data,
                                      nbytes), "bt_grouped_plan_norm")
    if device is None:
        device = problems[0]["x"].device
    dev = torch.from_numpy(host).to(device)
    return GroupedPlan(host, dev, keep)


def bt_gemm_grouped(plan: GroupedPlan, stream=None):
    torch = _torch()
    _check(lib().bt_gemm_grouped(_dev(plan.dev, torch.uint8, "plan"),
                                 plan.host.ctypes.data, _stream(stream)),
           "bt_gemm_grouped")


def bt_gemm_grouped_static(plan: GroupedPlan, stream=None):
    """bt_gemm_grouped with the kernels' scratch in the library's static
    device array (no allocation; calls on one GPU must not overlap)."""
    torch = _torch()
    _check(lib().bt_gemm_grouped_static(_dev(plan.dev, torch.uint8, "plan"),
                                        plan.host.ctypes.data,
                                        _stream(stream)),
           "bt_gemm_grouped_static")


def bt_read_probe(buf, sink, waves_per_cu: int = 8, groups: int = 2,
                  stream=None):
    """Stream-read a uint8 GPU buffer once (the read-ceiling probe); sink is
    an int32 GPU tensor with at least (compute units) * waves_per_cu
    elements."""
    torch = _torch()
    _check(lib().bt_read_probe(_dev(buf, torch.uint8, "buf"), buf.numel(),
                               _dev(sink, torch.int32, "sink"), sink.numel(),
                               int(waves_per_cu), int(groups),
                               _stream(stream)), "bt_read_probe")


def bt_mix_probe(buf, out, sink, waves_per_cu: int = 8, groups: int = 2,
                 burst: int = 1, stream=None):
    """Stream-read a uint8 GPU buffer once while writing the uint8 GPU
    buffer `out` once in bursts of `burst` 1 KiB pieces (the mixed
    read/write probe; out.numel() <= buf.numel(), both multiples of 1024);
    sink as for bt_read_probe."""
    torch = _torch()
    _check(lib().bt_mix_probe(_dev(buf, torch.uint8, "buf"), buf.numel(),
                              _dev(out, torch.uint8, "out"), out.numel(),
                              int(burst),
                              _dev(sink, torch.int32, "sink"), sink.numel(),
                              int(waves_per_cu), int(groups),
                              _stream(stream)), "bt_mix_probe")


class ChainPlan:
    """A chained launch's image (host and device copy); keeps its phase
    plans alive."""

    def __init__(self, host: np.ndarray, dev, plans):
        self.host = host
        self.dev = dev
        self._plans = plans


def bt_chain_plan(plans, device=None) -> ChainPlan:
    """plans: fused GroupedPlans (bt_grouped_plan_f32 / _norm), in the order
    their phases run."""
    torch = _torch()
    arr = (bt_chain_phase * len(plans))()
    for i, pl in enumerate(plans):
        arr[i] = bt_chain_phase(_dev(pl.dev, torch.uint8, "plan"),
                                pl.host.ctypes.data)
    nbytes = lib().bt_chain_plan_bytes(len(plans))
    if nbytes < 0:
        raise BtError(nbytes, "bt_chain_plan_bytes")
    host = np.zeros(nbytes, np.uint8)
    _check(lib().bt_chain_plan(arr, len(plans), host.ctypes.data, nbytes),
           "bt_chain_plan")
    if device is None:
        device = plans[0].dev.device
    return ChainPlan(host, torch.from_numpy(host).to(device), list(plans))


def bt_gemm_chain(chain: ChainPlan, stream=None):
    """All phases of the chain in one persistent launch."""
    torch = _torch()
    _check(lib().bt_gemm_chain(_dev(chain.dev, torch.uint8, "chain"),
                               chain.host.ctypes.data, _stream(stream)),
           "bt_gemm_chain")


def bt_chain_status(chain: ChainPlan) -> int:
    """The chain's status word (synchronizes): 0 after a complete launch,
    nonzero if a barrier wait gave up (outputs invalid)."""
    o = BT_CHAIN_STATUS_OFFSET
    return int(chain.dev[o:o + 4].cpu().numpy().view(np.int32)[0])
