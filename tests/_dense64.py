"""Independent fp64 dense brute force for the routed MXFP4 layer (tests only).

It does not call the oracle: E2M1 values come from the OCP MX v1.0 table fixture,
scales via numpy.ldexp, nibbles are split with numpy, and every expert is
evaluated densely with numpy matmuls in float64, then masked by the top-k one-hot.
"""
import os

import numpy as np

_GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def e2m1_fixture() -> np.ndarray:
    vals = np.empty(16, np.float64)
    with open(os.path.join(_GOLDEN, "e2m1_ocp_mx_v1.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            c, v = line.split()
            vals[int(c)] = float(v)
    return vals


def dequant64(codes: np.ndarray, scales: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """MXFP4 [rows][cols] -> float64 (NaN for scale 0xFF)."""
    table = e2m1_fixture()
    b = np.asarray(codes, np.uint8).reshape(rows, cols // 2)
    nib = np.empty((rows, cols), np.uint8)
    nib[:, 0::2] = b & 0xF
    nib[:, 1::2] = b >> 4
    s = np.asarray(scales, np.uint8).reshape(rows, cols // 32).astype(np.int64)
    s_full = np.repeat(s, 32, axis=1)
    with np.errstate(over="ignore", invalid="ignore"):
        v = np.ldexp(table[nib], s_full - 127)
        v[s_full == 255] = np.nan
    return v


def expert_mats64(codes_e, scales_e, H, I):
    mc, ms = I * H // 2, I * H // 32
    wg = dequant64(codes_e[:mc], scales_e[:ms], I, H)
    wu = dequant64(codes_e[mc:2 * mc], scales_e[ms:2 * ms], I, H)
    wd = dequant64(codes_e[2 * mc:], scales_e[2 * ms:], H, I)
    return wg, wu, wd


def layer64(x, w_router, experts, H, I, k, bias=None):
    """Returns (out, logits, idx, w) in float64 with selection by stable argsort."""
    x = np.asarray(x, np.float64)
    wr = np.asarray(w_router, np.float64)
    logits = x @ wr.T
    if bias is not None:
        logits = logits + np.asarray(bias, np.float64)
    T, E = logits.shape
    idx = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(logits, idx, 1)
    ex = np.exp(sel - sel[:, :1])
    w = ex / ex.sum(1, keepdims=True)
    mask = np.zeros((T, E))
    np.put_along_axis(mask, idx, w, 1)
    out = np.zeros((T, H))
    for e in range(E):
        if not mask[:, e].any():
            continue
        wg, wu, wd = expert_mats64(experts[e][0], experts[e][1], H, I)
        g = x @ wg.T
        u = x @ wu.T
        a = g / (1.0 + np.exp(-g)) * u
        y = a @ wd.T
        out += mask[:, e:e + 1] * y
    return out, logits, idx, w


def experts64(x, idx, w, experts, H, I):
    """Expert part with given routing in float64: out[t] = sum_j w[t,j] FFN_{idx[t,j]}(x[t])."""
    x = np.asarray(x, np.float64)
    idx = np.asarray(idx)
    w = np.asarray(w, np.float64)
    T, k = idx.shape
    out = np.zeros((T, H))
    for e in np.unique(idx):
        wg, wu, wd = expert_mats64(experts[e][0], experts[e][1], H, I)
        for t, j in zip(*np.nonzero(idx == e)):
            g = wg @ x[t]
            u = wu @ x[t]
            a = g / (1.0 + np.exp(-g)) * u
            out[t] += w[t, j] * (wd @ a)
    return out


def scale_ref64(x, experts, idx, w, H, I):
    """Magnitude scale A[t, n] = sum_j |w[t, j]| sum_i |h_j[i]| |Wd_j[n, i]| with
    h evaluated in float64 (for the elementwise error diagnostic); each distinct
    expert is decoded once."""
    x = np.asarray(x, np.float64)
    idx = np.asarray(idx)
    T = x.shape[0]
    out = np.zeros((T, H))
    for e in np.unique(idx):
        wg, wu, wd = expert_mats64(experts[e][0], experts[e][1], H, I)
        for t, j in zip(*np.nonzero(idx == e)):
            g = wg @ x[t]
            u = wu @ x[t]
            a = g / (1.0 + np.exp(-g)) * u
            out[t] += abs(w[t, j]) * (np.abs(wd) @ np.abs(a))
    return out
