"""Pins for the CPU oracle: each check compares it with something other than itself.

- E2M1 table: the OCP MX v1.0 table (fixture).
- E8M0 decode: PyTorch's float8_e8m0fnu conversion (a library routine).
- Dequant: all 16 codes x 256 scale bytes against numpy.ldexp of the fixture
  values; a hand-worked block for the nibble order.
- Logits: fp64 brute force within the textbook summation bound.
- Top-k: numpy stable argsort, with constructed ties, signed zeros, NaN, -inf.
- Softmax: closed forms for k = 1, 2; sum to one.
- Whole layer: dense fp64 brute force over all experts with a one-hot top-k mask
  (tests/_dense64.py, which never calls the oracle); closed-form special cases;
  permutation of expert storage; thread-count invariance.
- Expert part with given routing: dense fp64 brute force (repeated ids
  included) and the forward on the same routing.
- Magnitude scale of the elementwise error bar: fp64 numpy and a closed form.
- RMSNorm: constant-vector closed form and fp64.
- Packed-int8 rows: binary16 decode against numpy's float16 over all 65536
  patterns; int8 dequant bit-exact against fp64 products; the GEMV against
  fp64 within the textbook summation bound.
"""
import os
import shutil
import subprocess
import tempfile
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import _dense64 as d64

TOL = 2e-5


def bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


def normwise(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref), axis=-1)
    return np.max(np.abs(got - ref), axis=-1) / np.where(den == 0, 1.0, den)


# ------------------------------------------------------------------ formats

def test_e2m1_table_matches_ocp_fixture():
    t = oracle.e2m1_table()
    ref = d64.e2m1_fixture().astype(np.float32)
    assert np.array_equal(bits(t), bits(ref))  # -0.0 at code 8 included


def test_e8m0_matches_torch():
    s = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = s.view(torch.float8_e8m0fnu).to(torch.float32).numpy()
    got = np.array([oracle.e8m0_to_f32(i) for i in range(256)], np.float32)
    assert np.array_equal(bits(got[:255]), bits(ref[:255]))
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert bits(got[255:])[0] == 0x7FC00000


def enumeration_block():
    """256 rows (scale byte = row) x 32 columns (code = column % 16)."""
    cols = np.arange(32) % 16
    row_bytes = (cols[0::2] | (cols[1::2] << 4)).astype(np.uint8)
    codes = np.tile(row_bytes, 256)
    scales = np.arange(256, dtype=np.uint8)
    return codes, scales


def test_dequant_exhaustive_enumeration():
    codes, scales = enumeration_block()
    got = oracle.dequant(codes, scales, 256, 32)
    table = d64.e2m1_fixture()
    with np.errstate(over="ignore"):
        ref = np.ldexp(table[np.arange(32) % 16][None, :], (np.arange(256) - 127)[:, None]).astype(np.float32)
    ref[255, :] = np.frombuffer(np.uint32(0x7FC00000).tobytes(), np.float32)[0]
    assert np.array_equal(bits(got), bits(ref))
    # the cases the survey calls out explicitly
    assert bits(got[0, 1]) == 0x00200000          # 0.5 * 2^-127 = 2^-128, subnormal
    assert np.isposinf(got[254, 4]) and got[254, 3] == np.float32(1.5 * 2.0 ** 127)
    assert np.isposinf(got[253, 6]) and np.isneginf(got[253, 14])
    assert bits(got[127, 8]) == 0x80000000          # code 8 is -0.0


def test_dequant_nibble_order_worked_example(golden_dir):
    scale = None
    raw = vals = None
    with open(os.path.join(golden_dir, "mxfp4_block_worked_example.txt")) as f:
        for line in f:
            if line.startswith("scale"):
                scale = int(line.split()[1])
            elif line.startswith("bytes"):
                raw = np.array([int(b, 16) for b in line.split()[1:]], np.uint8)
            elif line.startswith("values"):
                vals = np.array([float(v) for v in line.split()[1:]], np.float32)
    got = oracle.dequant(raw, np.array([scale], np.uint8), 1, 32)[0]
    assert np.array_equal(bits(got), bits(vals))


def test_dequant_matches_dense64_on_random_matrices():
    rng = np.random.default_rng(7)
    rows, cols = 40, 96
    codes = rng.integers(0, 256, rows * cols // 2, dtype=np.uint8)
    scales = rng.integers(100, 150, rows * cols // 32, dtype=np.uint8)
    got = oracle.dequant(codes, scales, rows, cols)
    ref = d64.dequant64(codes, scales, rows, cols).astype(np.float32)
    assert np.array_equal(bits(got), bits(ref))


def test_bf16_widen_matches_torch():
    b = np.random.default_rng(1).integers(0, 65536, 4096, dtype=np.uint16)
    b = b[(b & 0x7F80) != 0x7F80]  # skip inf/NaN patterns (NaN payloads are not compared)
    got = oracle.bf16_to_f32(b)
    ref = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(bits(got), bits(ref))


# ------------------------------------------------------------------ router

def test_router_logits_within_summation_bound():
    rng = np.random.default_rng(3)
    T, E, H = 3, 5, 640
    x = rng.standard_normal((T, H)).astype(np.float32)
    w = (rng.standard_normal((E, H)) / np.sqrt(H)).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    got = oracle.router_logits(x, w, b).astype(np.float64)
    ref = x.astype(np.float64) @ w.astype(np.float64).T + b
    bound = (H + 1) * 2.0 ** -24 * (np.abs(x).astype(np.float64) @ np.abs(w).astype(np.float64).T + np.abs(b))
    assert np.all(np.abs(got - ref) <= bound)
    assert np.any(got != ref.astype(np.float32))  # really fp32, not a wider type


def test_router_bias_shifts_logits():
    x = np.zeros((1, 32), np.float32)
    w = np.ones((4, 32), np.float32)
    b = np.array([0.5, -1.0, 2.0, 0.0], np.float32)
    assert np.array_equal(oracle.router_logits(x, w, b)[0], b)


def stable_topk(l, k):
    return np.argsort(-np.asarray(l, np.float64), axis=1, kind="stable")[:, :k]


@pytest.mark.parametrize("seed", range(4))
def test_topk_random_matches_stable_argsort(seed):
    rng = np.random.default_rng(seed)
    l = rng.standard_normal((50, 37)).astype(np.float32)
    for k in (1, 5, 37):
        assert np.array_equal(oracle.topk(l, k), stable_topk(l, k))


def test_topk_constructed_ties():
    rng = np.random.default_rng(11)
    pool = np.array([1.0, 0.0, -0.0, -1.0, np.nan, -np.inf, np.inf, 0.5], np.float32)
    l = pool[rng.integers(0, len(pool), (200, 24))]
    l[0, :] = 3.0                       # all equal
    l[1, :] = np.nan                    # all NaN
    l[2, ::2], l[2, 1::2] = 0.0, -0.0   # signed zeros compare equal
    for k in (1, 4, 24):
        got = oracle.topk(l, k)
        ref = stable_topk(l, k)  # numpy sorts NaN last and keeps index order among ties
        assert np.array_equal(got, ref)
    assert np.array_equal(oracle.topk(l[:1], 5)[0], np.arange(5))


def test_softmax_closed_forms():
    rng = np.random.default_rng(5)
    l = rng.standard_normal((64, 9)).astype(np.float32) * 3
    idx1 = oracle.topk(l, 1)
    assert np.all(oracle.softmax_selected(l, idx1) == 1.0)
    idx2 = oracle.topk(l, 2)
    w2 = oracle.softmax_selected(l, idx2).astype(np.float64)
    l0 = np.take_along_axis(l, idx2[:, :1], 1)[:, 0].astype(np.float64)
    l1 = np.take_along_axis(l, idx2[:, 1:], 1)[:, 0].astype(np.float64)
    ref0 = 1.0 / (1.0 + np.exp(l1 - l0))
    assert np.all(np.abs(w2[:, 0] - ref0) <= 4 * 2.0 ** -24)
    assert np.all(np.abs(w2[:, 1] - (1 - ref0)) <= 4 * 2.0 ** -24)
    for k in (3, 9):
        idx = oracle.topk(l, k)
        w = oracle.softmax_selected(l, idx).astype(np.float64)
        assert np.all(np.abs(w.sum(1) - 1.0) <= k * 2.0 ** -23)
        assert np.all(np.diff(w, axis=1) <= 0)  # rank order = descending weight


# ------------------------------------------------------------------ whole layer

def tiny_case(seed, H=256, I=128, E=8, k=2, bias=False, T=1):
    w = synth.Workload("pin", 90 + seed, T, H, I, E, k, "f32", weight_seed=1000 + seed,
                       bias="none")
    x = synth.tokens_f32(w, range(T))
    wr = synth.router_w(w)
    c, s = synth.experts(w)
    ex = [(c[e * w.code_bytes_per_expert:(e + 1) * w.code_bytes_per_expert],
           s[e * w.scale_bytes_per_expert:(e + 1) * w.scale_bytes_per_expert]) for e in range(E)]
    b = None
    if bias:
        b = np.random.default_rng(seed).standard_normal(E).astype(np.float32)
    return x, wr, ex, b


@pytest.mark.parametrize("seed,shape", [
    (0, (256, 128, 8, 2)), (1, (256, 128, 8, 2)), (2, (256, 128, 8, 2)),
    (3, (64, 32, 5, 3)), (4, (96, 64, 16, 4)), (5, (32, 64, 4, 4)),
])
def test_layer_matches_dense_fp64(seed, shape):
    H, I, E, k = shape
    x, wr, ex, b = tiny_case(seed, H, I, E, k, bias=(seed % 2 == 1), T=3)
    out, logits, idx, w = oracle.moe_forward(x, wr, ex, H, I, k, bias=b)
    out64, l64, idx64, w64 = d64.layer64(x, wr, ex, H, I, k, bias=b)
    assert np.array_equal(idx, idx64)
    assert np.all(normwise(out, out64) <= TOL / 4)
    assert np.all(np.abs(w - w64) <= 4 * 2.0 ** -24 * np.maximum(1, w64))


def test_layer_special_cases():
    H, I, E, k = 64, 32, 6, 3
    x, wr, ex, _ = tiny_case(9, H, I, E, k)
    # x = 0: all logits 0 -> experts 0..k-1, weights 1/k, output +0
    out, logits, idx, w = oracle.moe_forward(np.zeros((1, H), np.float32), wr, ex, H, I, k)
    assert np.array_equal(idx[0], np.arange(k)) and np.all(w == np.float32(1.0 / k))
    assert np.all(bits(out) == 0)
    # all codes 0 -> zero weights -> output 0
    zero = [(np.zeros_like(c), s) for c, s in ex]
    out, *_ = oracle.moe_forward(x, wr, zero, H, I, k)
    assert np.all(out == 0)
    # codes 2 (value 1.0) with scale byte 127: every W is 1, so g = u = sum(x),
    # a = silu(S) * S and y[n] = I * a for every n and expert: out = I * a.
    ones = [(np.full_like(c, 0x22), np.full_like(s, 127)) for c, s in ex]
    out, *_ = oracle.moe_forward(x, wr, ones, H, I, k)
    S = float(np.sum(x.astype(np.float64)))
    a = S / (1 + np.exp(-S)) * S
    assert np.all(np.abs(out - I * a) <= TOL * abs(I * a))
    # a NaN scale byte in a selected expert poisons that token's output
    _, _, idx, _ = oracle.moe_forward(x, wr, ex, H, I, k)
    bad = list(ex)
    c, s = bad[idx[0, 0]]
    s = s.copy()
    s[0] = 0xFF
    bad[idx[0, 0]] = (c, s)
    out, *_ = oracle.moe_forward(x, wr, bad, H, I, k)
    assert np.all(np.isnan(out))


def test_layer_permutation_invariance():
    H, I, E, k = 96, 64, 12, 4
    x, wr, ex, b = tiny_case(21, H, I, E, k, bias=True, T=4)
    out, _, idx, w = oracle.moe_forward(x, wr, ex, H, I, k, bias=b)
    perm = np.random.default_rng(2).permutation(E)     # new slot q holds old expert perm[q]
    inv = np.argsort(perm)
    out_p, _, idx_p, w_p = oracle.moe_forward(x, wr[perm], [ex[perm[q]] for q in range(E)], H, I, k,
                                              bias=b[perm])
    assert np.array_equal(bits(out_p), bits(out))
    assert np.array_equal(perm[idx_p], idx)
    assert np.array_equal(bits(w_p), bits(w))
    assert np.array_equal(idx_p, inv[idx])


def test_layer_thread_count_invariance():
    H, I, E, k = 256, 128, 8, 2
    x, wr, ex, _ = tiny_case(33, H, I, E, k, T=5)
    a = oracle.moe_forward(x, wr, ex, H, I, k, nthreads=1)
    b = oracle.moe_forward(x, wr, ex, H, I, k, nthreads=4)
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))


def test_logits_override_drives_selection():
    H, I, E, k = 64, 32, 6, 2
    x, wr, ex, _ = tiny_case(41, H, I, E, k)
    lo = np.zeros((1, E), np.float32)
    lo[0, 4], lo[0, 1] = 2.0, 1.0
    out, logits, idx, w = oracle.moe_forward(x, wr, ex, H, I, k, logits_override=lo)
    assert np.array_equal(idx[0], [4, 1])
    assert np.array_equal(logits, lo)


def test_experts_given_routing_matches_dense_fp64():
    H, I, E, k, T = 96, 64, 7, 3, 4
    x, _, ex, _ = tiny_case(51, H, I, E, k, T=T)
    idx = np.array([[6, 0, 3], [0, 3, 6], [2, 2, 5], [4, 1, 1]], np.int32)  # repeated ids in rows 2, 3
    w = np.array([[0.5, 0.25, 0.25], [0.7, 0.2, 0.1], [0.3, 0.3, 0.4], [1.0, -0.5, 0.25]], np.float32)
    got = oracle.moe_experts(x, idx, w, ex, H, I, E)
    ref = d64.experts64(x, idx, w, ex, H, I)
    assert np.all(normwise(got, ref) <= TOL / 4)
    with pytest.raises(RuntimeError):
        oracle.moe_experts(x, np.full((T, k), E, np.int32), w, ex, H, I, E)  # ids must lie in [0, E)


def test_experts_given_routing_equals_forward_on_its_routing():
    """On the forward's own selection and weights the given-routing entry is
    the same computation, so the same bits (and the forward is pinned above)."""
    H, I, E, k = 256, 128, 8, 2
    x, wr, ex, b = tiny_case(52, H, I, E, k, bias=True, T=3)
    out, _, idx, w = oracle.moe_forward(x, wr, ex, H, I, k, bias=b)
    assert np.array_equal(bits(oracle.moe_experts(x, idx, w, ex, H, I, E)), bits(out))


def test_abs_scale_matches_dense_fp64():
    H, I, E, k, T = 128, 96, 6, 3, 3
    x, _, ex, _ = tiny_case(53, H, I, E, k, T=T)
    idx = np.array([[5, 0, 2], [1, 1, 4], [3, 2, 0]], np.int32)
    w = np.array([[0.6, 0.3, 0.1], [0.5, -0.25, 0.25], [0.2, 0.2, 0.6]], np.float32)
    got = oracle.moe_abs_scale(x, idx, w, ex, H, I, E)
    ref = d64.scale_ref64(x, ex, idx, w, H, I)  # h in fp64 here, fp32 in the oracle
    assert np.all(np.abs(got - ref) <= 1e-5 * ref)
    # a closed form: every weight 1 (codes 0x22, scale byte 127) gives g = u = S
    # = sum_h x[t, h], h = silu(S) * S for every i, and
    # A[t, n] = sum_j |w[t, j]| * I * |silu(S) * S| for every n
    ones = [(np.full_like(c, 0x22), np.full_like(s_, 127)) for c, s_ in ex]
    got = oracle.moe_abs_scale(x, idx, w, ones, H, I, E)
    S = x.astype(np.float64).sum(1)
    want = np.abs(w.astype(np.float64)).sum(1) * I * np.abs(S / (1 + np.exp(-S)) * S)
    assert np.all(np.abs(got - want[:, None]) <= 1e-5 * want[:, None])


def test_oracle_meets_elementwise_bar_against_fp64():
    """The elementwise reading of the 2e-5 bar, |oracle - exact| <= 2e-5 * A,
    holds for the fp32 oracle itself at the model's width (one token, one
    expert pair per rank), so a second fp32 implementation can be held to it."""
    H, I, E, k = 7168, 1536, 4, 2
    w_ = synth.Workload("pinw", 97, 1, H, I, E, k, "bf16", weight_seed=1097)
    x = synth.tokens_f32(w_, [0])
    c, s_ = synth.experts(w_)
    ce, se = w_.code_bytes_per_expert, w_.scale_bytes_per_expert
    ex = [(c[e * ce:(e + 1) * ce], s_[e * se:(e + 1) * se]) for e in range(E)]
    idx = np.array([[2, 0]], np.int32)
    w = np.array([[0.75, 0.25]], np.float32)
    got = oracle.moe_experts(x, idx, w, ex, H, I, E).astype(np.float64)
    ref = d64.experts64(x, idx, w, ex, H, I)
    A = oracle.moe_abs_scale(x, idx, w, ex, H, I, E)
    assert np.max(np.abs(got - ref) / A) <= TOL / 4


# ------------------------------------------------------------------ stack parts

def test_rmsnorm_closed_form_and_fp64():
    H = 7168
    c = np.float32(0.75)
    g = synth.gamma(synth.WORKLOADS["stack12"], 3)
    n = oracle.rmsnorm(np.full((1, H), c, np.float32), g, 1e-6)
    ref = c / np.sqrt(np.float64(c) ** 2 + 1e-6) * g.astype(np.float64)
    assert np.all(np.abs(n[0] - ref) <= 4 * 2.0 ** -24 * np.abs(ref))
    r = np.random.default_rng(0).standard_normal((3, H)).astype(np.float32)
    n = oracle.rmsnorm(r, g, 1e-6)
    r64 = r.astype(np.float64)
    ref = r64 / np.sqrt((r64 ** 2).mean(1, keepdims=True) + 1e-6) * g
    assert np.all(normwise(n, ref) <= 1e-5)


def test_residual_add():
    r = np.array([[1.0, -2.0, 3.0]], np.float32)
    assert np.array_equal(oracle.residual_add(r, np.array([[0.5, 0.5, -3.0]], np.float32)),
                          np.array([[1.5, -1.5, 0.0]], np.float32))


# ------------------------------------------------------------------ packed-int8 rows

def test_f16_decode_matches_numpy_all_patterns():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = h.view(np.float16).astype(np.float32)
    got = np.array([oracle.f16_to_f32(int(v)) for v in h], np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(bits(got)[~nan], bits(ref)[~nan])


def test_int8_dequant_exact_and_gemv_within_bound():
    rng = np.random.default_rng(12)
    N, K, T = 40, 320, 3
    q = rng.integers(-128, 128, (N, K), dtype=np.int64).astype(np.int8)
    s = (rng.uniform(0.5, 1.5, N) * 2.0 ** -9).astype(np.float16)
    s[3] = np.float16(6.0e-8)           # a subnormal scale
    s[4] = np.float16(-0.25)            # a negative scale
    w = oracle.int8_dequant(q, s.view(np.uint16))
    ref = q.astype(np.float64) * s.astype(np.float64)[:, None]
    assert np.array_equal(bits(w), bits(ref.astype(np.float32)))
    assert np.all(w.astype(np.float64) == ref)          # every product exact in fp32
    x = rng.standard_normal((T, K)).astype(np.float32)
    y = oracle.int8_gemv(q, s.view(np.uint16), x).astype(np.float64)
    y64 = x.astype(np.float64) @ ref.T
    bound = K * 2.0 ** -24 * (np.abs(x).astype(np.float64) @ np.abs(ref).T)
    assert np.all(np.abs(y - y64) <= bound)
    assert np.any(y != y64.astype(np.float32))          # really fp32, not a wider type


# ------------------------------------------------------------------ planted mistakes

MUTANTS = {
    "nibble order swapped": ("(byte >> (4 * (c & 1)))", "(byte >> (4 * (1 - (c & 1))))"),
    "scale bias off by one": ("ldexpf(1.0f, (int)s - 127)", "ldexpf(1.0f, (int)s - 126)"),
    "silu on up instead of gate": ("a[i] = (g / (1.0f + expf(-g))) * u;", "a[i] = (u / (1.0f + expf(-u))) * g;"),
    "softmax sign": ("ex[j] = expf(l[idx[t * k + j]] - m);", "ex[j] = expf(m - l[idx[t * k + j]]);"),
    "ties to higher index": ("return ia < ib;\n}", "return ia > ib;\n}"),
    "block axis wrong": ("scales[n * (cols / 32) + c / 32]", "scales[(n / 32) * (cols / 32) + c % (cols / 32)]"),
    "combine drops last rank": ("for (int64_t j = 0; j < k; ++j) acc = acc + w", "for (int64_t j = 0; j + 1 < k; ++j) acc = acc + w"),
    "fp16 exponent bias off by one": ("(int)ex - 15);", "(int)ex - 14);"),
}


def _pins_pass(lib_path):
    """Re-run a handful of the pins above against a given build."""
    saved = oracle._lib
    oracle._lib = None
    orig = oracle._LIB_PATH
    try:
        oracle._LIB_PATH = lib_path
        checks = [test_dequant_exhaustive_enumeration, test_f16_decode_matches_numpy_all_patterns,
                  lambda: test_dequant_nibble_order_worked_example(os.path.join(os.path.dirname(__file__), "golden")),
                  lambda: test_layer_matches_dense_fp64(0, (256, 128, 8, 2)),
                  lambda: test_layer_matches_dense_fp64(4, (96, 64, 16, 4)),
                  test_topk_constructed_ties, test_softmax_closed_forms]
        for chk in checks:
            try:
                chk()
            except AssertionError:
                return False
        return True
    finally:
        oracle._LIB_PATH = orig
        oracle._lib = saved


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle._SRC).read()
    assert src.count(old) >= 1, name
    mutated = src.replace(old, new, 1)
    cpath = tmp_path / "oracle_mutant.c"
    cpath.write_text(mutated)
    so = tmp_path / "liboracle_mutant.so"
    subprocess.check_call(["gcc", *oracle.CFLAGS, "-o", str(so), str(cpath), "-lm"])
    assert not _pins_pass(str(so)), "pins did not catch: " + name


def test_unmutated_build_passes_the_same_pins(tmp_path):
    so = tmp_path / "liboracle_copy.so"
    subprocess.check_call(["gcc", *oracle.CFLAGS, "-o", str(so), oracle._SRC, "-lm"])
    assert _pins_pass(str(so))
