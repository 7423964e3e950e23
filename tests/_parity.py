"""Comparison rules between the GPU library and the CPU oracle.

- Dequantised weights, top-k indices (given identical logits) and sort output:
  bit-exact.
- Layer outputs: per token, max_n |g - r| / max_n |r| <= 2e-5 (normwise; an
  elementwise relative error is ill-conditioned where outputs cancel to 0).
- Combine weights: |w_gpu - w_ora| <= 2 (k + 4) 2^-24 w_ora and the weights
  of each token sum to 1 within k * 2^-23.  Each side evaluates
  w_j = e_j / sum_i e_i with e_j = exp(l_j - l_0) on the same logits (l_j - l_0
  is the same fp32 difference on both): exp within 2 ulp, a sum of k positive
  terms within (k - 1) ulp in any order, the division within 1 ulp, so each
  side is within (k + 4) 2^-24 of the exact weight relative to it.
- Router logits: |l_gpu - l_ora| <= 2e-5 * sum_h |x_h W_eh| (+ |b_e|).
- Layer outputs, elementwise: |g_n - r_n| <= 2e-5 * A_n for every finite
  element, with A the oracle's magnitude scale (the layer on |x|, |W|, |w|;
  oracle.moe_abs_scale).
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


def elementwise_ratio(got, ref, A) -> float:
    """max over elements where ref and A are finite and A > 0 of |got - ref| / A."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    A = np.asarray(A, np.float64)
    m = np.isfinite(ref) & np.isfinite(A) & (A > 0)
    if not m.any():
        return 0.0
    with np.errstate(invalid="ignore"):
        return float(np.max(np.abs(got[m] - ref[m]) / A[m]))


def assert_elementwise(got, ref, A, tol=OUT_TOL):
    r = elementwise_ratio(got, ref, A)
    assert r <= tol, "elementwise error ratio %g > %g" % (r, tol)
    return r


def assert_layer_close(got, ref, x_f32, idx, w, experts, H, I, E, tol=OUT_TOL):
    """Both readings of the output bar on every token: normwise (primary) and
    elementwise against the oracle's magnitude scale.  Returns (normwise max,
    elementwise max)."""
    import oracle
    nw = assert_out_close(got, ref, tol)
    A = oracle.moe_abs_scale(x_f32, idx, w, experts, H, I, E)
    ew = assert_elementwise(got, ref, A, tol)
    return nw, ew


def weights_rel_err(w_gpu, w_ora) -> float:
    w_gpu = np.asarray(w_gpu, np.float64)
    w_ora = np.asarray(w_ora, np.float64)
    return float(np.max(np.abs(w_gpu - w_ora) / w_ora))


def assert_weights_close(w_gpu, w_ora, k):
    w_gpu = np.asarray(w_gpu, np.float64)
    w_ora = np.asarray(w_ora, np.float64)
    r = weights_rel_err(w_gpu, w_ora)
    assert r <= 2 * (k + 4) * 2.0 ** -24, "combine weights differ by %.3g relative (%.1f ulp)" % (r, r * 2 ** 24)
    assert np.all(np.abs(w_gpu.sum(-1) - 1.0) <= k * 2.0 ** -23)


def assert_logits_close(l_gpu, l_ora, x, wr, bias=None):
    scale = np.abs(np.asarray(x, np.float64)) @ np.abs(np.asarray(wr, np.float64)).T
    if bias is not None:
        scale = scale + np.abs(np.asarray(bias, np.float64))
    d = np.abs(np.asarray(l_gpu, np.float64) - np.asarray(l_ora, np.float64))
    assert np.all(d <= 2e-5 * scale), "logit error ratio %g" % (d / (scale + 1e-30)).max()


def bits(a):
    return np.ascontiguousarray(a).view(np.uint32)
