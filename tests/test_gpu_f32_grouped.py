"""fp32 activations in the grouped (prefill) form: from 9 tokens on, the
forward splits each fp32 activation into three exact bf16 terms laid along K
and runs the grouped MFMA GEMMs, so every expert's weights stream once per
batch instead of once per (token, rank) pair.

- against the oracle on every token (small shapes, several m-tile templates,
  ragged blocks) and on sampled tokens at the model's width;
- on fp32 x whose values are exact in bf16 the three-term form gives the
  bf16 form's values (its two extra terms are zeros);
- the layer stack (fp32 residual stream) with more than 8 tokens, layer by
  layer against the oracle;
- activations above bf16's largest finite value, and near 1e30 and 1e-30,
  in both the grouped and the per-token form.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import synth.device as sd
import mxfp4_routed_expert_fp32_amd as moe
from tests import _parity as P
from tests.test_gpu_parity import DEV, experts_host, pack_whole, run_forward

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("H,I,E,k,T", [(512, 256, 16, 4, 40), (1024, 512, 33, 6, 70), (256, 256, 4, 2, 9),
                                       (768, 256, 300, 16, 130)])
def test_f32_grouped_matches_oracle(H, I, E, k, T):
    w = synth.Workload("g32", 90, T, H, I, E, k, "f32", weight_seed=9500 + H + E)
    c, s, ex = experts_host(w)
    desc, codes, scales = pack_whole(w, c, s)
    x = sd.tokens(w, range(T))
    assert x.dtype == torch.float32
    wr = sd.router_w(w)
    bias = torch.from_numpy(np.random.default_rng(E).standard_normal(E).astype(np.float32)).to(DEV)
    out, logits, idx, wt = run_forward(desc, w, x, wr, bias, codes, scales, k)
    xf = synth.tokens_f32(w, range(T))
    r_out, _, r_idx, r_w = oracle.moe_forward(xf, wr.cpu().numpy(), ex, H, I, k, bias=bias.cpu().numpy(),
                                              logits_override=logits)
    assert np.array_equal(idx, r_idx)
    P.assert_weights_close(wt, r_w, k)
    P.assert_layer_close(out, r_out, xf, r_idx, r_w, ex, H, I, E)


def test_f32_grouped_model_width_sampled():
    """H = 7168, I = 1536, 24 experts, k = 16, 32 fp32 tokens: 512 pairs over
    24 experts (blocks of several m-tiles), six tokens against the oracle."""
    H, I, E, k, T = 7168, 1536, 24, 16, 32
    w = synth.Workload("g32m", 91, T, H, I, E, k, "f32", weight_seed=9700)
    c, s, ex = experts_host(w)
    desc, codes, scales = pack_whole(w, c, s)
    x = sd.tokens(w, range(T))
    wr = sd.router_w(w)
    out, logits, idx, wt = run_forward(desc, w, x, wr, None, codes, scales, k)
    sample = [0, 1, 7, 16, 30, 31]
    xf = synth.tokens_f32(w, sample)
    r_out, _, r_idx, r_w = oracle.moe_forward(xf, wr.cpu().numpy(), ex, H, I, k, logits_override=logits[sample])
    assert np.array_equal(idx[sample], r_idx)
    P.assert_layer_close(out[sample], r_out, xf, r_idx, r_w, ex, H, I, E)


def test_f32_grouped_equals_bf16_form_on_bf16_values():
    """fp32 x holding bf16 values, through the expert entry on one routing:
    the three-term grouped form (hi = x, mid = lo = 0) gives the values of the
    bf16 grouped form on the same x."""
    H, I, E, k, T = 1024, 512, 20, 4, 48
    w = synth.Workload("g32b", 92, T, H, I, E, k, "bf16", weight_seed=9800)
    c, s, _ = experts_host(w)
    desc, codes, scales = pack_whole(w, c, s)
    xb = sd.tokens(w, range(T))
    assert xb.dtype == torch.bfloat16
    _, _, idx, wt = run_forward(desc, w, xb, sd.router_w(w), None, codes, scales, k)
    idx_d, wt_d = torch.from_numpy(idx).to(DEV), torch.from_numpy(wt).to(DEV)
    outs = []
    for x in (xb, xb.float().contiguous()):
        out = torch.empty(T, H, dtype=torch.float32, device=DEV)
        ws = torch.empty(moe.workspace_bytes(desc, T, k), dtype=torch.uint8, device=DEV)
        moe.moe_mxfp4_experts(desc, x, idx_d, wt_d, codes, scales, k, out, ws)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])   # value equality (+0 == -0)


def test_stack_f32_tokens_grouped_layer_by_layer():
    """The layer stack with 12 tokens: its fp32 normalised rows take the
    three-term grouped form; two layers against the oracle layer by layer."""
    H, I, E, k, T = 512, 256, 16, 4, 12
    w = synth.Workload("stg", 93, T, H, I, E, k, "bf16", weight_seed=9900)
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


def test_f32_grouped_extreme_magnitudes():
    """fp32 activations far outside bf16's comfortable range, through the
    expert entry on fixed routes: token 0 holds values above bf16's largest
    finite value (3.3895e38, where the split keeps hi at that value and puts
    the rest in mid and lo), token 1 values near 1e30, token 2 values near
    1e-30, the rest N(0,1) times 1e29..1e31 per token.  Every weight has scale byte 27 (2^-100), so the
    large tokens still give finite h and outputs.  The grouped form (12
    tokens) and the per-token decode form both meet the bar against the
    oracle's given-routing entry."""
    H, I, E, k, T = 512, 256, 6, 3, 12
    w = synth.Workload("g32x", 94, T, H, I, E, k, "f32", weight_seed=9910)
    c, s, ex = experts_host(w)
    s[:] = 27
    ex = [(c[e * w.code_bytes_per_expert:(e + 1) * w.code_bytes_per_expert],
           s[e * w.scale_bytes_per_expert:(e + 1) * w.scale_bytes_per_expert]) for e in range(E)]
    desc, codes, scales = pack_whole(w, c, s)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((T, H)).astype(np.float32)
    x[0] = np.float32(3.395e38) * np.where(rng.random(H) < 0.5, -1.0, 1.0).astype(np.float32) \
        * (1.0 + 0.001 * rng.random(H)).astype(np.float32)
    assert np.all(np.isfinite(x[0])) and np.all(np.abs(x[0]) > np.float32(3.3895e38))
    x[1] *= np.float32(1e30)
    x[2] *= np.float32(1e-30)
    x[3:] *= (10.0 ** rng.uniform(29, 31, (T - 3, 1))).astype(np.float32)
    idx = np.array([[(t + j) % E for j in range(k)] for t in range(T)], np.int32)
    wts = np.array([[0.5, 0.3, 0.2]] * T, np.float32)
    r_out = oracle.moe_experts(x, idx, wts, ex, H, I, E)
    assert np.all(np.isfinite(r_out))
    xd = torch.from_numpy(x).to(DEV)
    idx_d, wts_d = torch.from_numpy(idx).to(DEV), torch.from_numpy(wts).to(DEV)
    out = torch.empty(T, H, dtype=torch.float32, device=DEV)
    ws = torch.empty(moe.workspace_bytes(desc, T, k), dtype=torch.uint8, device=DEV)
    moe.moe_mxfp4_experts(desc, xd, idx_d, wts_d, codes, scales, k, out, ws)          # grouped form
    torch.cuda.synchronize()
    P.assert_layer_close(out.cpu().numpy(), r_out, x, idx, wts, ex, H, I, E)
    one = torch.empty(1, H, dtype=torch.float32, device=DEV)
    ws1 = torch.empty(moe.workspace_bytes(desc, 1, k), dtype=torch.uint8, device=DEV)
    for t in (0, 1, 2):                                                               # decode form
        moe.moe_mxfp4_experts(desc, xd[t:t + 1], idx_d[t:t + 1], wts_d[t:t + 1], codes, scales, k, one, ws1)
        torch.cuda.synchronize()
        P.assert_layer_close(one.cpu().numpy(), r_out[t:t + 1], x[t:t + 1], idx[t:t + 1], wts[t:t + 1], ex, H,
                             I, E)
