"""GPU parity tests: the HIP library (through its C ABI) against the CPU oracle.

Bit-exact: dequantised weights (all 16 x 256 code/scale pairs and real-shape
experts), top-k indices given identical logits, and the expert sort.
Tolerance (tests/_parity.py): layer outputs, combine weights, logits.
End-to-end layer checks run the oracle on the GPU's own logits, so a near-tie
between the k-th and (k+1)-th logit cannot flip the selected set between the
two implementations; the logits themselves are checked separately.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import synth.device as sd
import mxfp4_routed_expert_fp32_amd as moe
from tests import _parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda"


def small_workload(H, I, E, k, seed, x_dtype="f32", bias="none"):
    return synth.Workload("t%d" % seed, 50 + seed, 1, H, I, E, k, x_dtype, weight_seed=7000 + seed, bias=bias)


def experts_host(w, layer=0):
    c, s = synth.experts(w, layer)
    ce, se = w.code_bytes_per_expert, w.scale_bytes_per_expert
    return c, s, [(c[e * ce:(e + 1) * ce], s[e * se:(e + 1) * se]) for e in range(w.E)]


def to_dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def pack_whole(w, c, s):
    desc = sd.desc_for(w)
    cb, sb = moe.packed_bytes(desc)
    codes = torch.empty(cb, dtype=torch.uint8, device=DEV)
    scales = torch.empty(sb, dtype=torch.uint8, device=DEV)
    moe.moe_mxfp4_pack(desc, to_dev_u8(c), to_dev_u8(s), 0, w.E, codes, scales)
    return desc, codes, scales


def run_forward(desc, w, x, wr, bias, codes, scales, k):
    T = x.shape[0]
    out = torch.empty(T, w.H, dtype=torch.float32, device=DEV)
    logits = torch.empty(T, w.E, dtype=torch.float32, device=DEV)
    idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    wt = torch.empty(T, k, dtype=torch.float32, device=DEV)
    ws = torch.empty(moe.workspace_bytes(desc, T, k), dtype=torch.uint8, device=DEV)
    moe.moe_mxfp4_forward(desc, x, wr, bias, codes, scales, k, out, ws, logits, idx, wt)
    torch.cuda.synchronize()
    return out.cpu().numpy(), logits.cpu().numpy(), idx.cpu().numpy(), wt.cpu().numpy()


# ------------------------------------------------------------------ dequant

def test_dequant_enumeration_bitexact():
    """Gate matrix [32][256]: block (r, b) has scale byte 8r + b, codes 0..15 twice."""
    w = small_workload(256, 32, 1, 1, 0)
    c, s, _ = experts_host(w)
    row = np.tile(np.array([0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE], np.uint8), 2 * 8)
    mc = w.I * w.H // 2
    c[:mc] = np.tile(row, w.I)
    s[:w.I * w.H // 32] = np.arange(256, dtype=np.uint8)
    desc, codes, scales = pack_whole(w, c, s)
    for m, (rows, cols) in enumerate([(w.I, w.H), (w.I, w.H), (w.H, w.I)]):
        out = torch.empty(rows, cols, dtype=torch.float32, device=DEV)
        moe.moe_mxfp4_dequant(desc, codes, scales, 0, m, out)
        torch.cuda.synchronize()
        mcb, msb = rows * cols // 2, rows * cols // 32
        ref = oracle.dequant(c[m * mc:m * mc + mcb], s[m * (w.I * w.H // 32):m * (w.I * w.H // 32) + msb], rows, cols)
        assert np.array_equal(P.bits(out.cpu().numpy()), P.bits(ref)), "matrix %d" % m
        assert_bf16_export_equals(desc, codes, scales, 0, m, ref)


def assert_bf16_export_equals(desc, codes, scales, e, m, ref):
    """The bf16-conversion export (the decode of the bf16 GEMV and both MFMA
    kernels) equals the oracle bit for bit wherever the oracle is not NaN, and
    is NaN exactly where the oracle is."""
    out = torch.empty(ref.shape, dtype=torch.float32, device=DEV)
    moe.moe_mxfp4_dequant_bf16(desc, codes, scales, e, m, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), (e, m)
    assert np.array_equal(P.bits(got)[~nan], P.bits(ref)[~nan]), (e, m)


def test_dequant_real_shape_bitexact():
    w = small_workload(7168, 1536, 3, 2, 1)
    c, s, ex = experts_host(w)
    # a few extreme scale bytes in expert 2: subnormal, overflow and NaN blocks
    se = w.scale_bytes_per_expert
    s[2 * se:2 * se + 6] = [0, 1, 253, 254, 255, 127]
    desc, codes, scales = pack_whole(w, c, s)
    for e in range(w.E):
        ce_, se_ = ex[e]
        if e == 2:
            se_ = s[2 * se:3 * se]
        for m, (rows, cols) in enumerate([(w.I, w.H), (w.I, w.H), (w.H, w.I)]):
            out = torch.empty(rows, cols, dtype=torch.float32, device=DEV)
            moe.moe_mxfp4_dequant(desc, codes, scales, e, m, out)
            torch.cuda.synchronize()
            mc, ms = w.I * w.H // 2, w.I * w.H // 32
            ref = oracle.dequant(ce_[m * mc:(m + 1) * mc], se_[m * ms:(m + 1) * ms], rows, cols)
            assert np.array_equal(P.bits(out.cpu().numpy()), P.bits(ref)), (e, m)
            assert_bf16_export_equals(desc, codes, scales, e, m, ref)


# ------------------------------------------------------------------ routing

@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (64, 896, 16), (33, 300, 7), (5, 64, 64), (3, 4096, 16)])
def test_topk_softmax_given_logits(T, E, k):
    rng = np.random.default_rng(T * 1000 + E)
    l = rng.standard_normal((T, E)).astype(np.float32)
    idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    wt = torch.empty(T, k, dtype=torch.float32, device=DEV)
    moe.moe_topk_softmax(torch.from_numpy(l).to(DEV), k, idx, wt)
    torch.cuda.synchronize()
    ref_idx = oracle.topk(l, k)
    assert np.array_equal(idx.cpu().numpy(), ref_idx)
    P.assert_weights_close(wt.cpu().numpy(), oracle.softmax_selected(l, ref_idx), k)


def test_topk_ties_signed_zero_nan_inf():
    rng = np.random.default_rng(3)
    pool = np.array([1.0, 0.0, -0.0, -1.0, np.nan, -np.inf, 0.5, 2.0], np.float32)
    T, E, k = 128, 96, 8
    l = pool[rng.integers(0, len(pool), (T, E))]
    l[0, :] = 3.0
    l[1, :] = np.nan
    l[2, ::2], l[2, 1::2] = 0.0, -0.0
    idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    wt = torch.empty(T, k, dtype=torch.float32, device=DEV)
    moe.moe_topk_softmax(torch.from_numpy(l).to(DEV), k, idx, wt)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), oracle.topk(l, k))


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_router_logits_within_bound(name):
    w = synth.WORKLOADS[name]
    x = sd.tokens(w, range(8))
    wr = sd.router_w(w)
    logits = torch.empty(8, w.E, dtype=torch.float32, device=DEV)
    moe.moe_router_logits(sd.desc_for(w), x, wr, None, logits)
    torch.cuda.synchronize()
    xf = synth.tokens_f32(w, range(8))
    wr_h = wr.cpu().numpy()
    P.assert_logits_close(logits.cpu().numpy(), oracle.router_logits(xf, wr_h), xf, wr_h)


@pytest.mark.parametrize("T,H,E", [(9, 256, 8), (130, 512, 33), (300, 7168, 896), (4096, 7168, 896)])
def test_router_mfma_logits_within_bound(T, H, E):
    """Many bf16 tokens take the MFMA router (fp32 weights as three bf16
    terms): ragged token and expert tiles, the decode model's shape and the
    4096-token prefill batch (sampled tokens)."""
    w = synth.Workload("rt", 64, T, H, 128, E, 2, "bf16", weight_seed=7600 + T + E)
    x = sd.tokens(w, range(T))
    wr = sd.router_w(w)
    b = np.random.default_rng(T).standard_normal(E).astype(np.float32)
    logits = torch.empty(T, E, dtype=torch.float32, device=DEV)
    moe.moe_router_logits(sd.desc_for(w), x, wr, torch.from_numpy(b).to(DEV), logits)
    torch.cuda.synchronize()
    rows = np.arange(T) if T <= 300 else np.unique(np.r_[0, 1, 127, 128, T - 1, np.random.default_rng(1).integers(0, T, 40)])
    xf = synth.tokens_f32(w, rows)
    wr_h = wr.cpu().numpy()
    got = logits.cpu().numpy()[rows]
    P.assert_logits_close(got, oracle.router_logits(xf, wr_h, bias=b), xf, wr_h, bias=b)


@pytest.mark.parametrize("T,H,E", [(64, 1024, 130), (200, 7168, 96), (37, 640, 40), (256, 512, 8)])
def test_router_split_k_matches_whole_tiles(T, H, E):
    """Up to 256 tokens, the forward runs the MFMA router's K slices in
    workgroups of their own and adds their partial sums in a second kernel;
    the router stage entry (no workspace) runs every slice of a tile in one
    workgroup.  Both add the same slice sums in the same order, so the logits
    are the same bits; H = 640 has an odd number of 128-wide chunks."""
    w = synth.Workload("rs", 66, T, H, 256, E, 2, "bf16", weight_seed=7800 + T + H)
    c, s, ex = experts_host(w)
    desc, codes, scales = pack_whole(w, c, s)
    x = sd.tokens(w, range(T))
    wr = sd.router_w(w)
    b = np.random.default_rng(T + 1).standard_normal(E).astype(np.float32)
    bias = torch.from_numpy(b).to(DEV)
    _, lf, _, _ = run_forward(desc, w, x, wr, bias, codes, scales, 2)
    logits = torch.empty(T, E, dtype=torch.float32, device=DEV)
    moe.moe_router_logits(desc, x, wr, bias, logits)
    torch.cuda.synchronize()
    ls = logits.cpu().numpy()
    assert np.array_equal(lf.view(np.uint32), ls.view(np.uint32))
    xf = synth.tokens_f32(w, range(T))
    wr_h = wr.cpu().numpy()
    P.assert_logits_close(lf, oracle.router_logits(xf, wr_h, bias=b), xf, wr_h, bias=b)


def test_sort_by_expert_matches_stable_sort():
    """One workgroup up to 1023 tokens, token blocks of 256 above (ragged last
    block, a skewed choice of experts, the largest E): both give numpy's
    stable argsort by expert."""
    rng = np.random.default_rng(9)
    for T, E, k, skew in [(1, 8, 2, False), (64, 896, 16, False), (4096, 896, 16, False), (130, 50, 5, False),
                          (1023, 40, 4, False), (1025, 40, 4, True), (5000, 4096, 8, False), (4097, 896, 16, True)]:
        if skew:  # most tokens pick the same few experts first
            idx = np.stack([np.r_[np.arange(3), 3 + rng.permutation(E - 3)[:k - 3]] if t % 5 else rng.permutation(E)[:k]
                            for t in range(T)]).astype(np.int32)
        else:
            idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        offs = torch.empty(E + 1, dtype=torch.int32, device=DEV)
        pairs = torch.empty(T * k, dtype=torch.int32, device=DEV)
        nws = moe.sort_workspace_bytes(E, T, k)
        assert (nws > 0) == (T >= 1024)
        ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=DEV)
        moe.moe_sort_by_expert(torch.from_numpy(idx).to(DEV), E, offs, pairs, ws)
        torch.cuda.synchronize()
        flat = idx.reshape(-1)
        order = np.argsort(flat, kind="stable")  # by expert, then pair id (= token, rank)
        assert np.array_equal(pairs.cpu().numpy(), order.astype(np.int32))
        counts = np.bincount(flat, minlength=E)
        assert np.array_equal(offs.cpu().numpy(), np.concatenate([[0], np.cumsum(counts)]).astype(np.int32))


@pytest.mark.parametrize("T,E,k", [(70, 40, 4), (130, 896, 16), (1100, 40, 4), (2048, 896, 16)])
def test_sort_repeated_and_out_of_range_ids(T, E, k):
    """Ids outside [0, E) are clamped into it and a row may name an expert
    twice; on both sort paths (one workgroup below 1024 tokens, blocks of 256
    above) the pair list is still numpy's stable argsort of the clamped ids (a
    permutation of the pairs), the offsets are their counts, and the words
    past the end of both outputs are untouched."""
    rng = np.random.default_rng(T + E)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    for t in rng.integers(0, T, max(4, T // 16)):
        j0, j1 = rng.integers(0, k, 2)
        idx[t, j1] = idx[t, j0]                   # a repeated id
    for t in rng.integers(0, T, max(4, T // 16)):
        idx[t, rng.integers(0, k)] = rng.choice([E, E + 7, -1, -100])
    idx[63, :2] = [E - 1, E + 2]                  # two ids that clamp to one expert, at a chunk's last token
    idx[64, :] = -3                               # a whole row clamped to expert 0
    guard = 64
    offs = torch.full((E + 1 + guard,), -7, dtype=torch.int32, device=DEV)
    pairs = torch.full((T * k + guard,), -7, dtype=torch.int32, device=DEV)
    nws = moe.sort_workspace_bytes(E, T, k)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=DEV)
    moe.moe_sort_by_expert(torch.from_numpy(idx).to(DEV), E, offs[:E + 1], pairs[:T * k], ws)
    torch.cuda.synchronize()
    flat = np.clip(idx.reshape(-1), 0, E - 1)
    p_h, o_h = pairs.cpu().numpy(), offs.cpu().numpy()
    assert np.array_equal(p_h[:T * k], np.argsort(flat, kind="stable").astype(np.int32))
    assert np.array_equal(o_h[:E + 1], np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    assert np.all(p_h[T * k:] == -7) and np.all(o_h[E + 1:] == -7)


# ------------------------------------------------------------------ whole layer, small shapes

def oracle_layer(x_f32, wr, ex, H, I, k, bias, logits_gpu):
    return oracle.moe_forward(x_f32, wr, ex, H, I, k, bias=bias, logits_override=logits_gpu)


@pytest.mark.parametrize("seed", range(6))
def test_forward_tiny_matches_oracle(seed):
    w = synth.WORKLOADS["tiny"]
    c, s, ex = experts_host(w)
    desc, codes, scales = pack_whole(w, c, s)
    ids = [seed]
    x = sd.tokens(w, ids)
    wr = sd.router_w(w)
    out, logits, idx, wt = run_forward(desc, w, x, wr, None, codes, scales, w.k)
    xf = synth.tokens_f32(w, ids)
    wr_h = wr.cpu().numpy()
    P.assert_logits_close(logits, oracle.router_logits(xf, wr_h), xf, wr_h)
    r_out, _, r_idx, r_w = oracle_layer(xf, wr_h, ex, w.H, w.I, w.k, None, logits)
    assert np.array_equal(idx, r_idx)
    P.assert_weights_close(wt, r_w, w.k)
    P.assert_layer_close(out, r_out, xf, r_idx, r_w, ex, w.H, w.I, w.E)


@pytest.mark.parametrize("H,I,E,k,T,xd", [(256, 128, 8, 2, 4, "f32"), (96, 64, 16, 4, 3, "bf16"),
                                           (64, 32, 6, 6, 2, "f32"), (512, 96, 33, 5, 7, "bf16"),
                                           (7168, 1536, 20, 16, 2, "bf16"),
                                           # down with K split across I/512 waves, ragged row ranges
                                           (160, 1024, 5, 2, 1, "f32"), (96, 2048, 6, 3, 3, "f32"),
                                           (64, 3072, 4, 2, 2, "f32"), (1056, 1536, 9, 4, 1, "bf16"),
                                           # decode-form GEMVs at other widths (bf16 x, one token or I % 128 != 0)
                                           (4096, 96, 5, 2, 3, "bf16"), (2048, 64, 4, 2, 1, "bf16"),
                                           # fp32 x: K halves across wave pairs, model width and an odd block count
                                           (7168, 1536, 20, 16, 2, "f32"), (1056, 160, 9, 4, 3, "f32"),
                                           # descriptor limits on the decode form: H = I = 8192 (the
                                           # widest gate/up and down GEMVs); E above 1024 with the largest
                                           # k (the selection's 64-slot form inside the gate/up kernel,
                                           # combine over four groups of 16 ranks)
                                           (8192, 8192, 2, 2, 1, "bf16"), (256, 128, 4096, 64, 2, "bf16"),
                                           (96, 64, 1500, 64, 1, "f32")])
def test_forward_small_shapes_matches_oracle(H, I, E, k, T, xd):
    w = synth.Workload("s", 60, T, H, I, E, k, xd, weight_seed=7100 + H + E)
    c, s, ex = experts_host(w)
    desc, codes, scales = pack_whole(w, c, s)
    x = sd.tokens(w, range(T))
    wr = sd.router_w(w)
    bias = torch.from_numpy(np.random.default_rng(E).standard_normal(E).astype(np.float32)).to(DEV)
    out, logits, idx, wt = run_forward(desc, w, x, wr, bias, codes, scales, k)
    xf = synth.tokens_f32(w, range(T))
    r_out, _, r_idx, r_w = oracle_layer(xf, wr.cpu().numpy(), ex, H, I, k, bias.cpu().numpy(), logits)
    assert np.array_equal(idx, r_idx)
    P.assert_weights_close(wt, r_w, k)
    P.assert_layer_close(out, r_out, xf, r_idx, r_w, ex, H, I, E)


@pytest.mark.parametrize("T,xd", [(5, "f32"), (1, "bf16"), (5, "bf16")])
def test_experts_entry_with_given_routing(T, xd):
    """Expert part on constructed routes (every token on the same experts,
    reversed rank order in one row) on the decode forms (fp32 x; one bf16
    token) and the prefill form (several bf16 tokens, H and I multiples of
    256), against the oracle's given-routing entry with the same weights."""
    w = synth.Workload("r", 61, T, 512, 256, 8, 3, xd, weight_seed=7300)
    c, s, ex = experts_host(w)
    desc, codes, scales = pack_whole(w, c, s)
    k = 3
    x = sd.tokens(w, range(T))
    idx = np.array([[7, 0, 3]] * T, np.int32)
    idx[T // 2] = [0, 3, 7]
    wts = np.array([[0.5, 0.25, 0.25]] * T, np.float32)
    wts[0] = [0.125, 0.625, 0.25]
    out = torch.empty(T, w.H, dtype=torch.float32, device=DEV)
    ws = torch.empty(moe.workspace_bytes(desc, T, k), dtype=torch.uint8, device=DEV)
    moe.moe_mxfp4_experts(desc, x, torch.from_numpy(idx).to(DEV), torch.from_numpy(wts).to(DEV), codes, scales,
                          k, out, ws)
    torch.cuda.synchronize()
    xf = synth.tokens_f32(w, range(T))
    r_out = oracle.moe_experts(xf, idx, wts, ex, w.H, w.I, w.E)
    P.assert_layer_close(out.cpu().numpy(), r_out, xf, idx, wts, ex, w.H, w.I, w.E)


@pytest.mark.parametrize("T,xd", [(6, "f32"), (70, "bf16"), (1100, "bf16")])
def test_experts_entry_repeated_and_out_of_range_ids(T, xd):
    """Routes that name one expert twice in a row, or ids outside [0, E) (which
    are clamped into it), on the decode form (fp32 x) and the prefill form
    (bf16 x; 70 tokens sort in one workgroup, 1100 tokens in blocks of 256):
    the output is the layer on the clamped routes, pair for pair."""
    H, I, E, k = 256, 256, 6, 3
    w = synth.Workload("dup", 71, T, H, I, E, k, xd, weight_seed=8200 + T)
    c, s, ex = experts_host(w)
    desc, codes, scales = pack_whole(w, c, s)
    rng = np.random.default_rng(T)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    idx[0] = [2, 2, 5]                 # a repeated id
    idx[1] = [E + 3, -4, E - 1]        # out of range both ways; E + 3 clamps onto E - 1
    idx[T - 1] = [1, 1, 1]
    if T > 64:
        idx[63] = [4, -1, 4]
        idx[64] = [0, 0, E]
    wts = rng.uniform(0.1, 1.0, (T, k)).astype(np.float32)
    x = sd.tokens(w, range(T))
    out = torch.empty(T, H, dtype=torch.float32, device=DEV)
    ws = torch.empty(moe.workspace_bytes(desc, T, k), dtype=torch.uint8, device=DEV)
    moe.moe_mxfp4_experts(desc, x, torch.from_numpy(idx).to(DEV), torch.from_numpy(wts).to(DEV), codes, scales,
                          k, out, ws)
    torch.cuda.synchronize()
    rows = np.unique(np.r_[0, 1, T - 1, np.arange(max(0, min(T, 70) - 8), min(T, 70)), rng.integers(0, T, 8)])
    xf = synth.tokens_f32(w, rows)
    cl = np.clip(idx[rows], 0, E - 1)
    r_out = oracle.moe_experts(xf, cl, wts[rows], ex, H, I, E)
    P.assert_layer_close(out.cpu().numpy()[rows], r_out, xf, cl, wts[rows], ex, H, I, E)


def test_forward_is_deterministic():
    w = synth.Workload("d", 62, 3, 512, 256, 16, 4, "bf16", weight_seed=7400)
    c, s, ex = experts_host(w)
    desc, codes, scales = pack_whole(w, c, s)
    x = sd.tokens(w, range(3))
    wr = sd.router_w(w)
    a = run_forward(desc, w, x, wr, None, codes, scales, 4)
    b = run_forward(desc, w, x, wr, None, codes, scales, 4)
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))


def test_rmsnorm_and_residual():
    H = 7168
    r = np.random.default_rng(4).standard_normal((3, H)).astype(np.float32)
    g = synth.gamma(synth.WORKLOADS["stack12"], 2)
    out = torch.empty(3, H, dtype=torch.float32, device=DEV)
    moe.moe_rmsnorm(torch.from_numpy(r).to(DEV), torch.from_numpy(g).to(DEV), 1e-6, out)
    torch.cuda.synchronize()
    P.assert_out_close(out.cpu().numpy(), oracle.rmsnorm(r, g, 1e-6), tol=1e-6)
    rd = torch.from_numpy(r).to(DEV)
    d = torch.from_numpy(r[::-1].copy()).to(DEV)
    moe.moe_residual_add(rd, d)
    torch.cuda.synchronize()
    assert np.array_equal(rd.cpu().numpy(), oracle.residual_add(r, r[::-1]))


# ------------------------------------------------------------------ prefill form (grouped GEMM on MFMA)

@pytest.mark.parametrize("H,I,E,k,T,hot", [(256, 256, 8, 2, 37, False), (512, 256, 16, 4, 65, False),
                                           (256, 512, 4, 2, 300, True), (1024, 768, 12, 3, 130, True),
                                           (768, 1280, 6, 2, 45, False),
                                           (8192, 256, 2, 1, 20, False), (256, 2816, 4, 2, 37, False)])
def test_prefill_grouped_gemm_matches_oracle(H, I, E, k, T, hot):
    """T > 1 with bf16 activations runs the sort + MFMA grouped GEMMs (H, I
    multiples of 256; an odd count of 256-wide K superchunks included); expert
    blocks are ragged, and `hot` makes one expert take more than 128 tokens.
    H = 8192 is the largest hidden size a layer may have (and the largest
    gate/up scale table in LDS); H = 256 has a single row tile, fewer than a
    down workgroup's run of tiles."""
    w = synth.Workload("g", 63, T, H, I, E, k, "bf16", weight_seed=7500 + H + E + T)
    c, s, ex = experts_host(w)
    desc, codes, scales = pack_whole(w, c, s)
    x = sd.tokens(w, range(T))
    wr = sd.router_w(w)
    b = np.zeros(E, np.float32)
    if hot:
        b[1] = 8.0  # expert 1 is selected by (nearly) every token
    bias = torch.from_numpy(b).to(DEV)
    out, logits, idx, wt = run_forward(desc, w, x, wr, bias, codes, scales, k)
    if hot:
        assert np.sum(idx == 1) > 128
    xf = synth.tokens_f32(w, range(T))
    P.assert_logits_close(logits, oracle.router_logits(xf, wr.cpu().numpy(), bias=b), xf, wr.cpu().numpy(), bias=b)
    # the forward's router (K slices in workgroups of their own up to 256 tokens,
    # summed in the top-k launch) gives the stage entry's whole-tile bits
    lg_stage = torch.empty(T, E, dtype=torch.float32, device=DEV)
    moe.moe_router_logits(desc, x, wr, bias, lg_stage)
    torch.cuda.synchronize()
    assert np.array_equal(P.bits(logits), P.bits(lg_stage.cpu().numpy()))
    r_out, _, r_idx, r_w = oracle_layer(xf, wr.cpu().numpy(), ex, H, I, k, b, logits)
    assert np.array_equal(idx, r_idx)
    P.assert_weights_close(wt, r_w, k)
    err, _ = P.assert_layer_close(out, r_out, xf, r_idx, r_w, ex, H, I, E)
    assert err < 1e-5, err


def test_prefill_token_batches_equal_separate_calls():
    """Past the grouped GEMMs' 32-bit offset limits the forward runs the
    prefill form over batches of tokens.  At H = I = 256, k = 8 a batch holds
    131071 tokens (k * I * 4 bytes of h terms per token below 1 GiB); 131071 +
    900 tokens take two batches.  Tokens are independent and each token's
    sums do not depend on which tokens share its expert blocks, so the output
    equals two separate calls bit for bit; sampled tokens of both batches are
    checked against the oracle."""
    H, I, E, k = 256, 256, 8, 8
    T1, T2 = 131071, 900
    T = T1 + T2
    w = synth.Workload("tb", 67, T, H, I, E, k, "bf16", weight_seed=7900)
    c, s, ex = experts_host(w)
    desc, codes, scales = pack_whole(w, c, s)
    x = sd.tokens(w, range(T))
    wr = sd.router_w(w)
    out, logits, idx, wt = run_forward(desc, w, x, wr, None, codes, scales, k)
    o1, l1, i1, w1 = run_forward(desc, w, x[:T1].contiguous(), wr, None, codes, scales, k)
    o2, l2, i2, w2 = run_forward(desc, w, x[T1:].contiguous(), wr, None, codes, scales, k)
    assert np.array_equal(logits.view(np.uint32), np.concatenate([l1, l2]).view(np.uint32))
    assert np.array_equal(idx, np.concatenate([i1, i2]))
    assert np.array_equal(out.view(np.uint32), np.concatenate([o1, o2]).view(np.uint32))
    rows = np.r_[0, 1, T1 - 1, T1, T1 + 1, T - 1, np.random.default_rng(3).integers(0, T, 12)]
    xf = synth.tokens_f32(w, rows)
    r_out, _, r_idx, r_w = oracle_layer(xf, wr.cpu().numpy(), ex, H, I, k, None, logits[rows])
    assert np.array_equal(idx[rows], r_idx)
    P.assert_weights_close(wt[rows], r_w, k)
    P.assert_layer_close(out[rows], r_out, xf, r_idx, r_w, ex, H, I, E)


def test_forward_max_tokens_sampled():
    """The largest token count a call accepts (2^20) on the prefill form,
    which runs it as several token batches; sampled tokens, including both
    ends, are checked against the oracle."""
    H, I, E, k = 256, 256, 16, 4
    T = 1 << 20
    w = synth.Workload("maxT", 68, T, H, I, E, k, "bf16", weight_seed=7950)
    c, s, ex = experts_host(w)
    desc, codes, scales = pack_whole(w, c, s)
    x = sd.tokens(w, range(T))
    wr = sd.router_w(w)
    out, logits, idx, wt = run_forward(desc, w, x, wr, None, codes, scales, k)
    del x
    rows = np.r_[0, 1, T // 2, T - 2, T - 1, np.random.default_rng(5).integers(0, T, 11)]
    xf = synth.tokens_f32(w, rows)
    r_out, _, r_idx, r_w = oracle_layer(xf, wr.cpu().numpy(), ex, H, I, k, None, logits[rows])
    assert np.array_equal(idx[rows], r_idx)
    P.assert_weights_close(wt[rows], r_w, k)
    P.assert_layer_close(out[rows], r_out, xf, r_idx, r_w, ex, H, I, E)


@pytest.mark.parametrize("H,I,E,k,T", [(512, 256, 16, 4, 3), (256, 128, 100, 3, 5), (1024, 256, 8, 2, 1),
                                       (512, 256, 33, 4, 2),  # E not a multiple of the router's experts per workgroup
                                       (256, 128, 2048, 32, 2)])  # the 64-slot selection on fp32 activations
def test_stack_small_matches_oracle_layer_by_layer(H, I, E, k, T):
    """The layer stack (RMSNorm inside each layer's router kernel, fp32
    residual stream) on small shapes: two layers against the oracle layer by
    layer on the GPU's logits.  E > H/4 leaves some router workgroups without
    a slice of the normalised rows to write; T > 1 runs the 4-token tiles."""
    w = synth.Workload("st", 68, T, H, I, E, k, "bf16", weight_seed=8000 + H + E)
    desc = sd.desc_for(w)
    packed, exs = [], []
    for l in range(2):
        c, s, ex = experts_host(w, l)
        packed.append(pack_whole(w, c, s)[1:])
        exs.append(ex)
    wrs = [sd.router_w(w, l) for l in range(2)]
    gam = [sd.gamma(w, l) for l in range(2)]
    x = sd.tokens(w, range(T))
    resid = torch.empty(T, H, dtype=torch.float32, device=DEV)
    ws = torch.empty(moe.stack_workspace_bytes(desc, T, k), dtype=torch.uint8, device=DEV)
    moe.moe_mxfp4_stack_forward(desc, [p[0] for p in packed], [p[1] for p in packed], wrs, None, gam, w.eps, x, k,
                                resid, ws)
    torch.cuda.synchronize()
    got = resid.cpu().numpy()
    r = synth.tokens_f32(w, range(T))
    for l in range(2):
        n = oracle.rmsnorm(r, gam[l].cpu().numpy(), w.eps)
        lg = torch.empty(T, E, dtype=torch.float32, device=DEV)
        moe.moe_router_logits(desc, torch.from_numpy(n).to(DEV), wrs[l], None, lg)
        torch.cuda.synchronize()
        o, *_ = oracle.moe_forward(n, wrs[l].cpu().numpy(), exs[l], H, I, k, logits_override=lg.cpu().numpy())
        r = oracle.residual_add(r, o)
    P.assert_out_close(got, r)


def test_grouped_stages_equal_forward_and_skip_malformed_blocks():
    """The prefill form run stage by stage through its own entry points (sort,
    expert blocks, grouped gate/up, grouped down, combine) gives the forward's
    output bit for bit; the block list matches a host recomputation from the
    sort's offsets; blocks naming no valid expert or pair range are skipped."""
    H, I, E, k, T = 512, 256, 16, 4, 165
    w = synth.Workload("gs", 65, T, H, I, E, k, "bf16", weight_seed=7700)
    c, s, ex = experts_host(w)
    desc, codes, scales = pack_whole(w, c, s)
    x = sd.tokens(w, range(T))
    wr = sd.router_w(w)
    b = np.zeros(E, np.float32)
    b[3] = 8.0                                   # expert 3 takes every token: > 128 pairs, two blocks
    bias = torch.from_numpy(b).to(DEV)
    out, logits, idx, wt = run_forward(desc, w, x, wr, bias, codes, scales, k)
    Pn = T * k
    offs = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    pairs = torch.empty(Pn, dtype=torch.int32, device=DEV)
    moe.moe_sort_by_expert(torch.from_numpy(idx).to(DEV), E, offs, pairs)
    mb = moe.max_expert_blocks(E, Pn)
    blocks = torch.zeros(mb, 4, dtype=torch.int32, device=DEV)
    nb = torch.zeros(1, dtype=torch.int32, device=DEV)
    moe.moe_expert_blocks(offs, Pn, blocks, nb)
    hterm = torch.empty(2, Pn, I, dtype=torch.bfloat16, device=DEV)
    y = torch.empty(Pn, H, dtype=torch.float32, device=DEV)
    moe.moe_mxfp4_grouped_gate_up(desc, x, k, pairs, blocks, nb, codes, scales, hterm)
    moe.moe_mxfp4_grouped_down(desc, hterm, pairs, blocks, nb, codes, scales, y)
    o2 = torch.empty(T, H, dtype=torch.float32, device=DEV)
    moe.moe_combine(y, torch.from_numpy(wt).to(DEV), o2)
    torch.cuda.synchronize()
    assert np.array_equal(P.bits(o2.cpu().numpy()), P.bits(out))

    offs_h = offs.cpu().numpy()
    want = []
    for e in range(E):
        for m0 in range(offs_h[e], offs_h[e + 1], 128):
            want.append([e, m0, min(128, offs_h[e + 1] - m0), 0])
    n = int(nb.cpu().item())
    assert n == len(want) and len(want) > E - 1
    assert np.array_equal(blocks.cpu().numpy()[:n], np.array(want, np.int32))

    bad = torch.tensor([[E, 0, 4, 0], [0, Pn - 2, 4, 0], [1, 0, 0, 0], [-1, 0, 1, 0], [2, 0, 129, 0]],
                       dtype=torch.int32, device=DEV)
    nbad = torch.tensor([5], dtype=torch.int32, device=DEV)
    y2 = torch.full((Pn, H), 7.0, dtype=torch.float32, device=DEV)
    h2 = torch.full((2, Pn, I), 3.0, dtype=torch.bfloat16, device=DEV)
    moe.moe_mxfp4_grouped_gate_up(desc, x, k, pairs, bad, nbad, codes, scales, h2)
    moe.moe_mxfp4_grouped_down(desc, hterm, pairs, bad, nbad, codes, scales, y2)
    torch.cuda.synchronize()
    assert bool((y2 == 7.0).all()) and bool((h2 == 3.0).all())


# ------------------------------------------------------------------ extreme scale bytes through the forward

def hostile_layer(H=512):
    """A layer whose routed experts carry extreme E8M0 scale bytes.

    Expert 1 (every token selects it, through its bias):
      - gate/up blocks with scale bytes 0 and 1 (subnormal weights);
      - gate row 6, block 3: scale 253 with codes of magnitude <= 1.5 (finite
        weights near 2^126);
      - down row 10, block 0: scale 255 (NaN), so output column 10 is NaN;
      - down row 11, block 1: scale 254 with one code 2.0 (+inf weight);
      - down row 12, block 2: scale 253 with one code 4.0 and one -4.0 (+inf
        and -inf weights);
      - down row 13, block 3: scale 253 with codes of magnitude <= 1.5.
    Expert 5 (only token 2 selects it, through x[2][0]): gate row 0, block 0
    has scale 255, so every h of that pair, and token 2's whole output, is NaN.
    Activations are N(0,1) * 2^-20 (exact in bf16), so no finite sum comes near
    the fp32 overflow threshold and every non-finite output is fixed by the
    weights alone, whatever the summation order.  H = 1024 takes the K-split
    gate/up GEMV (one wave per 1024 columns) on the decode forms; H = 512 the
    row-per-wave GEMVs."""
    I, E, k, T = 256, 8, 2, 5
    w = synth.Workload("hs", 69, T, H, I, E, k, "bf16", weight_seed=8100 if H == 512 else 8100 + H)
    c, s, _ = experts_host(w)
    ce, se = w.code_bytes_per_expert, w.scale_bytes_per_expert
    mc, ms = I * H // 2, I * H // 32

    def blk(e, m, row, b, cols):  # (first code byte, scale byte) of block b of a row
        return e * ce + m * mc + row * (cols // 2) + 16 * b, e * se + m * ms + row * (cols // 32) + b

    def set_scale(e, m, row, b, cols, v, codes=None, small=False):
        cb, sb = blk(e, m, row, b, cols)
        s[sb] = v
        if small:
            c[cb:cb + 16] &= 0xBB            # clear bit 2 of both nibbles: |value| <= 1.5
        if codes is not None:
            c[cb:cb + 16] = 0
            for col, code in codes:          # col within the block
                c[cb + col // 2] |= np.uint8(code << (4 * (col & 1)))

    set_scale(1, 0, 3, 0, H, 0)
    set_scale(1, 0, 4, 1, H, 1)
    set_scale(1, 1, 5, 2, H, 0)
    set_scale(1, 1, 7, 3, H, 1)
    set_scale(1, 0, 6, 3, H, 253, small=True)
    set_scale(1, 2, 10, 0, I, 255)
    set_scale(1, 2, 11, 1, I, 254, codes=[(8, 4)])             # +2.0 * 2^127 = +inf
    set_scale(1, 2, 12, 2, I, 253, codes=[(6, 6), (11, 14)])   # +4.0 and -4.0 times 2^126
    set_scale(1, 2, 13, 3, I, 253, small=True)
    set_scale(5, 0, 0, 0, H, 255)
    ex = [(c[e * ce:(e + 1) * ce], s[e * se:(e + 1) * se]) for e in range(E)]
    x = synth.tokens_f32(w, range(T)) * np.float32(2.0 ** -20)
    x[:, 0] = 0.0
    x[2, 0] = 2.0 ** -10
    wr = synth.router_w(w)
    wr[:, 0] = 0.0
    wr[5, :] = 0.0
    wr[5, 0] = 1.0                           # logit_5 = x[t][0]: 2^-10 for token 2, 0 otherwise
    b = np.full(E, 1e-4, np.float32)         # the other logits are about 1e-4 +- 1e-6
    b[1], b[5] = 8.0, 0.0
    return w, c, s, ex, x, wr, b


@pytest.mark.parametrize("H", [512, 1024])
@pytest.mark.parametrize("form", ["decode_bf16", "decode_f32", "prefill_mfma"])
def test_forward_extreme_scale_bytes(form, H):
    """Scale bytes 0, 1, 253, 254 and 255 in selected experts, through each
    kernel form of the forward: NaN and +-inf land where the oracle puts them
    and every finite element meets both readings of the output bar.  The
    decode forms multiply h in fp32, so every element's class matches exactly.
    The prefill form feeds h to the bf16 matrix cores as two terms (hi + lo);
    an infinite weight times a zero or opposite-signed lo term is NaN, so there
    an element the oracle gives as +-inf may come out NaN (never finite, never
    the other sign)."""
    w, c, s, ex, x, wr, b = hostile_layer(H)
    desc, codes, scales = pack_whole(w, c, s)
    wr_d, b_d = torch.from_numpy(wr).to(DEV), torch.from_numpy(b).to(DEV)
    xb_bits = synth.f32_to_bf16_bits(x)
    assert np.array_equal(synth.bf16_bits_to_f32(xb_bits), x)    # x is exact in bf16
    xb = torch.from_numpy(xb_bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    if form == "decode_bf16":   # one token per call
        parts = [run_forward(desc, w, xb[t:t + 1], wr_d, b_d, codes, scales, w.k) for t in range(w.T)]
        out, logits, idx, wt = (np.concatenate([p[i] for p in parts]) for i in range(4))
    elif form == "decode_f32":
        out, logits, idx, wt = run_forward(desc, w, torch.from_numpy(x).to(DEV), wr_d, b_d, codes, scales, w.k)
    else:
        out, logits, idx, wt = run_forward(desc, w, xb, wr_d, b_d, codes, scales, w.k)
    r_out, _, r_idx, r_w = oracle.moe_forward(x, wr, ex, w.H, w.I, w.k, bias=b, logits_override=logits)
    assert np.array_equal(idx, r_idx)
    assert np.all(idx[:, 0] == 1) and idx[2, 1] == 5 and np.all(np.delete(idx[:, 1], 2) != 5)
    assert np.all(np.isnan(r_out[2])) and np.all(np.isnan(out[2]))
    assert np.all(np.isnan(r_out[:, 10])) and np.any(np.isinf(r_out[:, 11:13]))
    fin = np.isfinite(r_out)
    assert np.array_equal(np.isfinite(out), fin)
    assert np.all(np.isnan(out[np.isnan(r_out)]))
    inf = np.isinf(r_out)
    if form == "prefill_mfma":
        same = (out[inf] == r_out[inf]) | np.isnan(out[inf])
        assert np.all(same)
    else:
        assert np.array_equal(P.bits(out[inf]), P.bits(r_out[inf]))
    A = oracle.moe_abs_scale(x, r_idx, r_w, ex, w.H, w.I, w.E)
    for t in range(w.T):
        f = fin[t]
        if f.any():
            P.assert_out_close(out[t][f][None], r_out[t][f][None])
            P.assert_elementwise(out[t][f], r_out[t][f], A[t][f])


@pytest.mark.parametrize("H", [512, 1024])
def test_forward_extreme_scale_bytes_f32_grouped(H):
    """The hostile layer with its five fp32 tokens given twice (10 tokens), so
    the forward takes the grouped form on three exact bf16 terms of x: NaN
    where the oracle has NaN (tokens 2 and 7 whole, column 10), +-inf or NaN
    where it has +-inf (as on the bf16 grouped form), and every finite
    element within both readings of the bar."""
    w, c, s, ex, x, wr, b = hostile_layer(H)
    desc, codes, scales = pack_whole(w, c, s)
    x2 = np.concatenate([x, x])
    out, logits, idx, wt = run_forward(desc, w, torch.from_numpy(x2).to(DEV), torch.from_numpy(wr).to(DEV),
                                       torch.from_numpy(b).to(DEV), codes, scales, w.k)
    r_out, _, r_idx, r_w = oracle.moe_forward(x2, wr, ex, w.H, w.I, w.k, bias=b, logits_override=logits)
    assert np.array_equal(idx, r_idx)
    assert np.all(idx[:, 0] == 1) and idx[2, 1] == 5 and idx[7, 1] == 5
    assert np.all(np.isnan(r_out[[2, 7]])) and np.all(np.isnan(out[[2, 7]]))
    fin = np.isfinite(r_out)
    assert np.array_equal(np.isfinite(out), fin)
    assert np.all(np.isnan(out[np.isnan(r_out)]))
    inf = np.isinf(r_out)
    assert inf.any() and np.all((out[inf] == r_out[inf]) | np.isnan(out[inf]))
    A = oracle.moe_abs_scale(x2, r_idx, r_w, ex, w.H, w.I, w.E)
    for t in range(x2.shape[0]):
        f = fin[t]
        if f.any():
            P.assert_out_close(out[t][f][None], r_out[t][f][None])
            P.assert_elementwise(out[t][f], r_out[t][f], A[t][f])


def test_down_stage_wide_inter_many_pairs():
    """The decode-form down projection (K split across I/512 waves) with many
    pairs at the widest row of partial sums: H = 7168, I = 4096, 2048 pairs.
    The grid target alone would give each workgroup all 7168 rows (7168 * 8
    partials, over the LDS a workgroup may have); the rows are capped and split
    into more workgroups.  Sampled pairs against the oracle's dequantised
    matrix in fp64."""
    H, I, E, P_ = 7168, 4096, 3, 2048
    w = synth.Workload("wd", 72, 1, H, I, E, 1, "f32", weight_seed=8300)
    c, s, ex = experts_host(w)
    desc, codes, scales = pack_whole(w, c, s)
    rng = np.random.default_rng(17)
    pe = rng.integers(0, E, P_).astype(np.int32)
    h = (rng.standard_normal((P_, I)) * 0.01).astype(np.float32)
    y = torch.empty(P_, H, dtype=torch.float32, device=DEV)
    moe.moe_mxfp4_down(desc, torch.from_numpy(h).to(DEV), torch.from_numpy(pe).to(DEV), codes, scales, y)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    assert np.all(np.isfinite(got))
    mc, ms = I * H // 2, I * H // 32
    for e in range(E):
        rows = np.nonzero(pe == e)[0]
        rows = np.unique(np.r_[rows[:2], rows[-2:], rng.choice(rows, 2)])
        wd = oracle.dequant(ex[e][0][2 * mc:], ex[e][1][2 * ms:], H, I).astype(np.float64)
        ref = h[rows].astype(np.float64) @ wd.T
        A = np.abs(h[rows]).astype(np.float64) @ np.abs(wd).T
        P.assert_out_close(got[rows], ref)
        P.assert_elementwise(got[rows], ref, A)


@pytest.mark.parametrize("T,E,k,xd", [(1, 896, 16, "bf16"), (3, 300, 7, "f32"), (2, 4096, 64, "bf16")])
def test_gate_up_select_stage(T, E, k, xd):
    """The selecting gate/up stage (the decode forward's first expert kernel):
    its selection and weights equal moe_topk_softmax on the same logits, and
    its h equals the routes-given gate/up stage on that selection, bit for bit."""
    H, I = 512, 256
    w = synth.Workload("gs2", 74, T, H, I, E, k, xd, weight_seed=8500 + E)
    c, s, ex = experts_host(w)
    desc, codes, scales = pack_whole(w, c, s)
    x = sd.tokens(w, range(T))
    lg = torch.from_numpy(np.random.default_rng(E).standard_normal((T, E)).astype(np.float32)).to(DEV)
    idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    wt = torch.empty(T, k, dtype=torch.float32, device=DEV)
    h = torch.empty(T * k, I, dtype=torch.float32, device=DEV)
    moe.moe_mxfp4_gate_up_select(desc, x, lg, k, codes, scales, idx, wt, h)
    idx2 = torch.empty(T, k, dtype=torch.int32, device=DEV)
    wt2 = torch.empty(T, k, dtype=torch.float32, device=DEV)
    moe.moe_topk_softmax(lg, k, idx2, wt2)
    h2 = torch.empty(T * k, I, dtype=torch.float32, device=DEV)
    moe.moe_mxfp4_gate_up(desc, x, idx2.reshape(-1), k, codes, scales, h2)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), idx2.cpu().numpy())
    assert np.array_equal(P.bits(wt.cpu().numpy()), P.bits(wt2.cpu().numpy()))
    assert np.array_equal(P.bits(h.cpu().numpy()), P.bits(h2.cpu().numpy()))


def hostile_logit_rows(E, k, rng):
    """Rows that take every branch of the selection: random; all equal (more
    than 64 candidates); all NaN and fewer than k numbers (no bound); ties
    with signed zeros, NaN and -inf; a tie at the top; -inf with a few
    numbers; one huge and the rest tiny."""
    rows = [rng.standard_normal(E)]
    rows.append(np.full(E, 0.5))
    rows.append(np.full(E, np.nan))
    r = np.full(E, np.nan)
    r[rng.choice(E, min(E, max(1, k // 2)), replace=False)] = rng.standard_normal(min(E, max(1, k // 2)))
    rows.append(r)
    pool = np.array([1.0, 0.0, -0.0, -1.0, np.nan, -np.inf, 0.5, 2.0])
    rows.append(pool[rng.integers(0, len(pool), E)])
    r = rng.standard_normal(E)
    r[rng.choice(E, min(E, 5), replace=False)] = 10.0
    rows.append(r)
    r = np.full(E, -np.inf)
    r[rng.choice(E, min(E, k + 3), replace=False)] = rng.standard_normal(min(E, k + 3))
    rows.append(r)
    r = rng.standard_normal(E) * 1e-30
    r[E // 2] = 3e38
    rows.append(r)
    return np.stack(rows).astype(np.float32)


@pytest.mark.parametrize("H,E,k,xd", [(7168, 896, 16, "bf16"), (7168, 896, 16, "f32"), (2048, 1024, 16, "bf16"),
                                      (3072, 1000, 64, "f32"), (2048, 8, 2, "bf16"), (8192, 130, 7, "bf16")])
def test_gate_up_select_stage_split_k(H, E, k, xd):
    """The selecting gate/up stage in its K-split form (H a multiple of 1024,
    E <= 1024: the decode forward's form at the model's width), where all
    the workgroup's waves share the selection: on hostile logit rows (ties,
    signed zeros, NaN, -inf, more than 64 candidates, fewer than k numbers)
    its selection and weights equal moe_topk_softmax bit for bit, and its h
    equals the routes-given stage on that selection."""
    I = 64
    rng = np.random.default_rng(E + H + k)
    lg_h = hostile_logit_rows(E, k, rng)
    T = lg_h.shape[0]
    w = synth.Workload("gsk", 75, T, H, I, E, k, xd, weight_seed=8600 + E + H)
    c, s, _ = experts_host(w)
    desc, codes, scales = pack_whole(w, c, s)
    x = sd.tokens(w, range(T))
    lg = torch.from_numpy(lg_h).to(DEV)
    idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    wt = torch.empty(T, k, dtype=torch.float32, device=DEV)
    h = torch.empty(T * k, I, dtype=torch.float32, device=DEV)
    moe.moe_mxfp4_gate_up_select(desc, x, lg, k, codes, scales, idx, wt, h)
    idx2 = torch.empty(T, k, dtype=torch.int32, device=DEV)
    wt2 = torch.empty(T, k, dtype=torch.float32, device=DEV)
    moe.moe_topk_softmax(lg, k, idx2, wt2)
    h2 = torch.empty(T * k, I, dtype=torch.float32, device=DEV)
    moe.moe_mxfp4_gate_up(desc, x, idx2.reshape(-1), k, codes, scales, h2)
    torch.cuda.synchronize()
    assert np.array_equal(idx2.cpu().numpy(), oracle.topk(lg_h, k))
    assert np.array_equal(idx.cpu().numpy(), idx2.cpu().numpy())
    assert np.array_equal(P.bits(wt.cpu().numpy()), P.bits(wt2.cpu().numpy()))
    assert np.array_equal(P.bits(h.cpu().numpy()), P.bits(h2.cpu().numpy()))
