"""Comparison rules between the GPU library and the CPU oracle.

- Dequantised weights, top-k indices (given identical logits) and sort output:
  bit-exact.
- Layer outputs: per token, max_n |g - r| / max_n |r| <= 2e-5 (normwise; an
  elementwise relative error is ill-conditioned where outputs cancel to 0).
- Combine weights: |w_gpu - w_ora| <= 4 * 2^-24 * max(1, w) and the weights
  of each token sum to 1 within k * 2^-23.
- Router logits: |l_gpu - l_ora| <= 2e-5 * sum_h |x_h W_eh| (+ |b_e|).
"""
import numpy as np

OUT_TOL = 2e-5


def normwise_err(got, ref) -> np.ndarray:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref), axis=-1)
    return np.max(np.abs(got - ref), axis=-1) / np.where(den == 0, 1.0, den)


def assert_out_close(got, ref, tol=OUT_TOL):
    err = normwise_err(got, ref)
    assert np.all(np.isfinite(got)), "non-finite GPU output"
    assert np.all(err <= tol), "normwise error %s > %g" % (err.max(), tol)
    return float(err.max())


def assert_weights_close(w_gpu, w_ora, k):
    w_gpu = np.asarray(w_gpu, np.float64)
    w_ora = np.asarray(w_ora, np.float64)
    assert np.all(np.abs(w_gpu - w_ora) <= 4 * 2.0 ** -24 * np.maximum(1.0, w_ora))
    assert np.all(np.abs(w_gpu.sum(-1) - 1.0) <= k * 2.0 ** -23)


def assert_logits_close(l_gpu, l_ora, x, wr, bias=None):
    scale = np.abs(np.asarray(x, np.float64)) @ np.abs(np.asarray(wr, np.float64)).T
    if bias is not None:
        scale = scale + np.abs(np.asarray(bias, np.float64))
    d = np.abs(np.asarray(l_gpu, np.float64) - np.asarray(l_ora, np.float64))
    assert np.all(d <= 2e-5 * scale), "logit error ratio %g" % (d / (scale + 1e-30)).max()


def bits(a):
    return np.ascontiguousarray(a).view(np.uint32)
