"""Seeded synthetic inputs for the routed MXFP4 MoE layer.

A module of its own, shared by the tests, the benchmark and the CPU reference.
It holds none of the layer's arithmetic: it generates code bytes, scale bytes,
activations, router weights, router biases and RMSNorm gains with the shapes and
distributions of the workloads, from a counter-based generator (``synth.c``),
so any expert or token can be regenerated alone.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lock = threading.Lock()
_lib = None

BASE_SEED = 0x4D4F45  # "MOE"

# tensor ids inside the stream key (kept in step with synth.c)
T_X, T_ROUTER_W, T_GATE_CODES, T_UP_CODES, T_DOWN_CODES = 1, 2, 3, 4, 5
T_GATE_SCALES, T_UP_SCALES, T_DOWN_SCALES, T_GAMMA, T_ZIPF_PERM = 6, 7, 8, 9, 10
T_INT8_CODES, T_INT8_SCALES = 11, 12


def build(force: bool = True) -> str:
    """Compile libsynth.so with gcc (OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
                               "-ffp-contract=off", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build(force=True)
            L = ctypes.CDLL(_LIB_PATH)
            u64, u32, i64, vp = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64, ctypes.c_void_p
            L.synth_key.restype = u64
            L.synth_key.argtypes = [u64, u32, u32, u64]
            L.synth_draw.restype = u64
            L.synth_draw.argtypes = [u64, u64]
            L.synth_bytes.argtypes = [u64, u64, vp]
            L.synth_uint_range.argtypes = [u64, u64, u32, u32, vp]
            L.synth_normal_f32.argtypes = [u64, u64, ctypes.c_double, ctypes.c_double, vp]
            L.synth_uniform_f32.argtypes = [u64, u64, ctypes.c_double, ctypes.c_double, vp]
            L.synth_f32_to_bf16.argtypes = [vp, u64, vp]
            L.synth_expert.argtypes = [u64, u32, i64, i64, u64, vp, vp]
            L.synth_experts.argtypes = [u64, u32, i64, i64, u64, u64, vp, vp]
            _lib = L
    return _lib


def _ptr(a) -> int:
    if isinstance(a, np.ndarray):
        assert a.flags["C_CONTIGUOUS"]
        return a.ctypes.data
    return int(a)  # raw address (e.g. a pinned torch tensor's data_ptr())


def key(seed: int, layer: int, tensor: int, item: int) -> int:
    return lib().synth_key(seed, layer, tensor, item)


def draw(k: int, i: int) -> int:
    return lib().synth_draw(k, i)


def random_bytes(k: int, n: int) -> np.ndarray:
    out = np.empty(n, np.uint8)
    lib().synth_bytes(k, n, out.ctypes.data)
    return out


def uint_range(k: int, n: int, lo: int, span: int) -> np.ndarray:
    out = np.empty(n, np.uint8)
    lib().synth_uint_range(k, n, lo, span, out.ctypes.data)
    return out


def normal_f32(k: int, n: int, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    out = np.empty(n, np.float32)
    lib().synth_normal_f32(k, n, mean, std, out.ctypes.data)
    return out


def uniform_f32(k: int, n: int, lo: float, hi: float) -> np.ndarray:
    out = np.empty(n, np.float32)
    lib().synth_uniform_f32(k, n, lo, hi, out.ctypes.data)
    return out


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, np.float32)
    out = np.empty(a.shape, np.uint16)
    lib().synth_f32_to_bf16(a.ctypes.data, a.size, out.ctypes.data)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening: the 16 bits become the top half of an fp32."""
    return (np.ascontiguousarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------- workloads

@dataclass(frozen=True)
class Workload:
    name: str
    wid: int          # workload id, part of the token stream key
    T: int            # tokens per call
    H: int            # hidden
    I: int            # expert intermediate
    E: int            # routed experts
    k: int            # top-k
    x_dtype: str      # "f32" | "bf16"
    layers: int = 1
    bias: str = "none"   # "none" | "zipf"
    zipf_s: float = 1.1
    eps: float = 1e-6    # RMSNorm epsilon (stack only)
    weight_seed: int = BASE_SEED

    @property
    def code_bytes_per_expert(self) -> int:
        return 3 * self.I * self.H // 2

    @property
    def scale_bytes_per_expert(self) -> int:
        return 3 * self.I * self.H // 32

    @property
    def expert_bytes(self) -> int:
        return self.code_bytes_per_expert + self.scale_bytes_per_expert


K3_SEED = BASE_SEED + 1
WORKLOADS = {
    "tiny": Workload("tiny", 0, 1, 256, 128, 8, 2, "f32"),
    "decode": Workload("decode", 1, 1, 7168, 1536, 896, 16, "bf16", weight_seed=K3_SEED),
    "decode64_zipf": Workload("decode64_zipf", 2, 64, 7168, 1536, 896, 16, "bf16", bias="zipf",
                              weight_seed=K3_SEED),
    "prefill4096": Workload("prefill4096", 3, 4096, 7168, 1536, 896, 16, "bf16", weight_seed=K3_SEED),
    "stack12": Workload("stack12", 4, 1, 7168, 1536, 896, 16, "bf16", layers=12, weight_seed=K3_SEED),
}


def tokens_f32(w: Workload, token_ids, std: float = 1.0) -> np.ndarray:
    """Activations ~N(0,1), one independent stream per token id. For bf16
    workloads the values are rounded to bf16 (RNE) and returned widened to fp32."""
    rows = []
    for t in token_ids:
        v = normal_f32(key(w.weight_seed, 0, T_X, (w.wid << 32) | int(t)), w.H, 0.0, std)
        rows.append(v)
    x = np.stack(rows) if rows else np.zeros((0, w.H), np.float32)
    if w.x_dtype == "bf16":
        x = bf16_bits_to_f32(f32_to_bf16_bits(x))
    return x


def tokens_bf16_bits(w: Workload, token_ids) -> np.ndarray:
    return f32_to_bf16_bits(tokens_f32(w, token_ids))


def router_w(w: Workload, layer: int = 0) -> np.ndarray:
    """fp32 [E, H] ~ N(0, 1/H) (1/H is the variance)."""
    std = 1.0 / np.sqrt(w.H)
    out = np.empty((w.E, w.H), np.float32)
    L = lib()
    for e in range(w.E):
        L.synth_normal_f32(key(w.weight_seed, layer, T_ROUTER_W, e), w.H, 0.0, std, out[e].ctypes.data)
    return out


def zipf_rank(w: Workload, layer: int = 0) -> np.ndarray:
    """rank[e] in 1..E from a seeded Fisher-Yates shuffle."""
    kk = key(w.weight_seed, layer, T_ZIPF_PERM, 0)
    perm = np.arange(w.E)
    for i in range(w.E - 1, 0, -1):
        j = int((draw(kk, i) >> 32) * (i + 1) >> 32)
        perm[i], perm[j] = perm[j], perm[i]
    rank = np.empty(w.E, np.int64)
    rank[perm] = np.arange(1, w.E + 1)
    return rank


def router_bias(w: Workload, layer: int = 0):
    """None, or for "zipf": b_e = Phi^-1(pi_e), pi_e = min(1, c * rank^-s / sum) with c
    chosen so that sum(pi) = k; against router logits that are ~N(0,1) this makes
    expert popularity follow a Zipf law over a seeded rank order."""
    if w.bias == "none":
        return None
    from scipy.special import ndtri
    rank = zipf_rank(w, layer).astype(np.float64)
    p = rank ** (-w.zipf_s)
    p /= p.sum()
    lo, hi = 0.0, 1e6
    for _ in range(200):
        c = 0.5 * (lo + hi)
        if np.minimum(1.0, c * p).sum() < w.k:
            lo = c
        else:
            hi = c
    pi = np.clip(np.minimum(1.0, hi * p), 1e-9, 1 - 1e-9)
    return ndtri(pi).astype(np.float32)


def gamma(w: Workload, layer: int) -> np.ndarray:
    """RMSNorm gain per layer, uniform in [0.5, 1.5)."""
    return uniform_f32(key(w.weight_seed, layer, T_GAMMA, 0), w.H, 0.5, 1.5)


def expert(w: Workload, e: int, layer: int = 0):
    """(codes, scales) of one expert in the logical layout."""
    c = np.empty(w.code_bytes_per_expert, np.uint8)
    s = np.empty(w.scale_bytes_per_expert, np.uint8)
    lib().synth_expert(w.weight_seed, layer, w.H, w.I, e, c.ctypes.data, s.ctypes.data)
    return c, s


def experts_into(w: Workload, layer: int, e0: int, count: int, codes_out, scales_out) -> None:
    """Experts [e0, e0+count) back to back into two host buffers (numpy arrays or
    raw addresses of pinned memory)."""
    lib().synth_experts(w.weight_seed, layer, w.H, w.I, e0, count, _ptr(codes_out), _ptr(scales_out))


def experts(w: Workload, layer: int = 0, e0: int = 0, count=None):
    count = w.E - e0 if count is None else count
    c = np.empty(count * w.code_bytes_per_expert, np.uint8)
    s = np.empty(count * w.scale_bytes_per_expert, np.uint8)
    experts_into(w, layer, e0, count, c, s)
    return c, s


def int8_rows(seed: int, N: int, K: int):
    """Packed-int8 rows for the resident-spine GEMV: q [N, K] int8 uniform over
    -127..127, and one fp16 row scale [N] (as uint16 bits) uniform in
    [0.5, 1.5) * 2^-12, so that a row dotted with N(0,1) activations of
    K = 7168 is of order 1."""
    k = key(seed, 0, T_INT8_CODES, (N << 20) | K)
    q = (uint_range(k, N * K, 0, 255).astype(np.int16) - 127).astype(np.int8).reshape(N, K)
    sc = uniform_f32(key(seed, 0, T_INT8_SCALES, (N << 20) | K), N, 0.5, 1.5) * np.float32(2.0 ** -12)
    return q, sc.astype(np.float16).view(np.uint16)
