"""CPU oracle for the routed MXFP4 MoE layer (ctypes wrapper around oracle.c).

TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The GPU library never calls it, and
it shares no code with the GPU library.  It reads the logical MXFP4 layout:
per expert, codes gate [I][H/2] | up [I][H/2] | down [H][I/2] and scales
gate [I][H/32] | up [I][H/32] | down [H][I/32], low nibble = even element.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

CFLAGS = ["-O2", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off", "-std=c11"]


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc: no fast-math, no FMA contraction."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build(force=True)
            L = ctypes.CDLL(_LIB_PATH)
            i64, vp, f32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
            L.oracle_e2m1_table.argtypes = [vp]
            L.oracle_e8m0_to_f32.argtypes = [ctypes.c_uint8]
            L.oracle_e8m0_to_f32.restype = f32
            L.oracle_dequant.argtypes = [vp, vp, i64, i64, vp]
            L.oracle_bf16_to_f32.argtypes = [vp, i64, vp]
            L.oracle_router_logits.argtypes = [vp, i64, i64, vp, vp, i64, vp]
            L.oracle_topk.argtypes = [vp, i64, i64, i64, vp]
            L.oracle_softmax_selected.argtypes = [vp, vp, i64, i64, i64, vp]
            L.oracle_moe_forward.argtypes = [i64, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp,
                                             vp, vp, vp, ctypes.c_int]
            L.oracle_moe_forward.restype = ctypes.c_int
            L.oracle_moe_experts.argtypes = [i64, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, ctypes.c_int]
            L.oracle_moe_experts.restype = ctypes.c_int
            L.oracle_moe_abs_scale.argtypes = [i64, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, ctypes.c_int]
            L.oracle_moe_abs_scale.restype = ctypes.c_int
            L.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
            L.oracle_f16_to_f32.restype = f32
            L.oracle_int8_dequant.argtypes = [vp, vp, i64, i64, vp]
            L.oracle_int8_gemv.argtypes = [vp, vp, i64, i64, vp, i64, vp]
            L.oracle_rmsnorm.argtypes = [vp, vp, f32, i64, i64, vp]
            L.oracle_residual_add.argtypes = [vp, vp, i64]
            _lib = L
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _p(a):
    return None if a is None else a.ctypes.data


def e2m1_table() -> np.ndarray:
    t = np.empty(16, np.float32)
    lib().oracle_e2m1_table(t.ctypes.data)
    return t


def e8m0_to_f32(s: int) -> float:
    return lib().oracle_e8m0_to_f32(s)


def dequant(codes, scales, rows: int, cols: int) -> np.ndarray:
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    assert codes.size == rows * cols // 2 and scales.size == rows * cols // 32
    out = np.empty((rows, cols), np.float32)
    lib().oracle_dequant(codes.ctypes.data, scales.ctypes.data, rows, cols, out.ctypes.data)
    return out


def bf16_to_f32(bits) -> np.ndarray:
    bits = _c(bits, np.uint16)
    out = np.empty(bits.shape, np.float32)
    lib().oracle_bf16_to_f32(bits.ctypes.data, bits.size, out.ctypes.data)
    return out


def router_logits(x, w_router, bias=None) -> np.ndarray:
    x = _c(x, np.float32)
    w_router = _c(w_router, np.float32)
    T, H = x.shape
    E = w_router.shape[0]
    b = None if bias is None else _c(bias, np.float32)
    out = np.empty((T, E), np.float32)
    lib().oracle_router_logits(x.ctypes.data, T, H, w_router.ctypes.data, _p(b), E, out.ctypes.data)
    return out


def topk(logits, k: int) -> np.ndarray:
    logits = _c(logits, np.float32)
    T, E = logits.shape
    idx = np.empty((T, k), np.int32)
    lib().oracle_topk(logits.ctypes.data, T, E, k, idx.ctypes.data)
    return idx


def softmax_selected(logits, idx) -> np.ndarray:
    logits = _c(logits, np.float32)
    idx = _c(idx, np.int32)
    T, E = logits.shape
    k = idx.shape[1]
    w = np.empty((T, k), np.float32)
    lib().oracle_softmax_selected(logits.ctypes.data, idx.ctypes.data, T, E, k, w.ctypes.data)
    return w


def moe_forward(x, w_router, experts, H: int, I: int, k: int, bias=None, logits_override=None,
                nthreads: int = 0):
    """Full layer.  ``experts`` maps expert id -> (codes, scales) uint8 arrays in the
    logical layout (only selected experts are required; a list of E pairs also
    works).  Returns (out, logits, idx, w)."""
    x = _c(x, np.float32)
    w_router = _c(w_router, np.float32)
    T = x.shape[0]
    E = w_router.shape[0]
    assert x.shape[1] == H and w_router.shape[1] == H
    cp = (ctypes.c_void_p * E)()
    sp = (ctypes.c_void_p * E)()
    keep = []
    items = experts.items() if isinstance(experts, dict) else enumerate(experts)
    for e, pair in items:
        if pair is None:
            continue
        c = _c(pair[0], np.uint8)
        s = _c(pair[1], np.uint8)
        assert c.size == 3 * I * H // 2 and s.size == 3 * I * H // 32
        keep += [c, s]
        cp[e] = c.ctypes.data
        sp[e] = s.ctypes.data
    b = None if bias is None else _c(bias, np.float32)
    lo = None if logits_override is None else _c(logits_override, np.float32)
    out = np.empty((T, H), np.float32)
    logits = np.empty((T, E), np.float32)
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    rc = lib().oracle_moe_forward(T, H, I, E, k, x.ctypes.data, w_router.ctypes.data, _p(b),
                                  ctypes.cast(cp, ctypes.c_void_p), ctypes.cast(sp, ctypes.c_void_p),
                                  _p(lo), out.ctypes.data, logits.ctypes.data, idx.ctypes.data,
                                  w.ctypes.data, nthreads)
    if rc != 0:
        raise RuntimeError("oracle_moe_forward failed with %d" % rc)
    return out, logits, idx, w


def _expert_ptrs(experts, E, H, I):
    cp = (ctypes.c_void_p * E)()
    sp = (ctypes.c_void_p * E)()
    keep = []
    items = experts.items() if isinstance(experts, dict) else enumerate(experts)
    for e, pair in items:
        if pair is None:
            continue
        c = _c(pair[0], np.uint8)
        s = _c(pair[1], np.uint8)
        assert c.size == 3 * I * H // 2 and s.size == 3 * I * H // 32
        keep += [c, s]
        cp[e] = c.ctypes.data
        sp[e] = s.ctypes.data
    return cp, sp, keep


def moe_experts(x, idx, w, experts, H: int, I: int, E: int, nthreads: int = 0) -> np.ndarray:
    """Expert part with the routing given: out[t] = sum_j w[t,j] FFN_{idx[t,j]}(x[t])."""
    x = _c(x, np.float32)
    idx = _c(idx, np.int32)
    w = _c(w, np.float32)
    T, k = idx.shape
    assert x.shape == (T, H) and w.shape == (T, k)
    cp, sp, keep = _expert_ptrs(experts, E, H, I)
    out = np.empty((T, H), np.float32)
    rc = lib().oracle_moe_experts(T, H, I, E, k, x.ctypes.data, idx.ctypes.data, w.ctypes.data,
                                  ctypes.cast(cp, ctypes.c_void_p), ctypes.cast(sp, ctypes.c_void_p),
                                  out.ctypes.data, nthreads)
    if rc != 0:
        raise RuntimeError("oracle_moe_experts failed with %d" % rc)
    return out


def moe_abs_scale(x, idx, w, experts, H: int, I: int, E: int, nthreads: int = 0) -> np.ndarray:
    """Per-element magnitude scale A [T][H] (float64) for the given routing:
    A[t, n] = sum_j |w[t, j]| sum_i |h_j[i]| |Wd_j[n, i]| (see oracle.c)."""
    x = _c(x, np.float32)
    idx = _c(idx, np.int32)
    w = _c(w, np.float32)
    T, k = idx.shape
    cp, sp, keep = _expert_ptrs(experts, E, H, I)
    A = np.empty((T, H), np.float64)
    rc = lib().oracle_moe_abs_scale(T, H, I, E, k, x.ctypes.data, idx.ctypes.data, w.ctypes.data,
                                    ctypes.cast(cp, ctypes.c_void_p), ctypes.cast(sp, ctypes.c_void_p),
                                    A.ctypes.data, nthreads)
    if rc != 0:
        raise RuntimeError("oracle_moe_abs_scale failed with %d" % rc)
    return A


def f16_to_f32(h: int) -> float:
    return lib().oracle_f16_to_f32(h)


def int8_dequant(q, s_f16_bits) -> np.ndarray:
    """W[n, k] = q[n, k] * s[n] for packed int8 rows q [N, K] and fp16 scale bits s [N]."""
    q = _c(q, np.int8)
    s = _c(s_f16_bits, np.uint16)
    N, K = q.shape
    out = np.empty((N, K), np.float32)
    lib().oracle_int8_dequant(q.ctypes.data, s.ctypes.data, N, K, out.ctypes.data)
    return out


def int8_gemv(q, s_f16_bits, x) -> np.ndarray:
    """y [T, N] = x [T, K] . W^T with W = q * s (fp32, ascending k)."""
    q = _c(q, np.int8)
    s = _c(s_f16_bits, np.uint16)
    x = _c(x, np.float32)
    N, K = q.shape
    T = x.shape[0]
    y = np.empty((T, N), np.float32)
    lib().oracle_int8_gemv(q.ctypes.data, s.ctypes.data, N, K, x.ctypes.data, T, y.ctypes.data)
    return y


def rmsnorm(r, gamma, eps: float) -> np.ndarray:
    r = _c(r, np.float32)
    gamma = _c(gamma, np.float32)
    T, H = r.shape
    out = np.empty_like(r)
    lib().oracle_rmsnorm(r.ctypes.data, gamma.ctypes.data, eps, T, H, out.ctypes.data)
    return out


def residual_add(r, d) -> np.ndarray:
    r = np.array(r, np.float32, copy=True)
    d = _c(d, np.float32)
    lib().oracle_residual_add(r.ctypes.data, d.ctypes.data, r.size)
    return r
