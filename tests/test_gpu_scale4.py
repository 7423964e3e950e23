"""The lossless scale4 side-car: encoding, both dequant exports, the decode
GEMV stages and the forward are bit-identical to the 8-bit scale table;
rows whose scales span more than 15 are reported (the layer keeps the 8-bit
table); many bf16 tokens, which the 8-bit layer runs on the MFMA form, take
the decode form on scale4 and are checked against the oracle."""
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


def layer_with_extreme_rows(H, I, E, k, seed):
    """A layer (host arrays) where some rows have all their scale bytes at the
    extremes: all 0 (subnormal weights), all 254 (mostly infinite), all 255
    (NaN), and 240..255 (base 240, the largest deltas)."""
    w = synth.Workload("s4", 80, 1, H, I, E, k, "bf16", weight_seed=seed)
    c, s = synth.experts(w)
    se, ms = w.scale_bytes_per_expert, I * H // 32
    s = s.copy()
    e = 1
    s[e * se + 2 * (H // 32):e * se + 3 * (H // 32)] = 0                 # gate row 2: all 0
    dn = e * se + 2 * ms
    s[dn + 5 * (I // 32):dn + 6 * (I // 32)] = 254                       # down row 5: all 254
    s[dn + 6 * (I // 32):dn + 7 * (I // 32)] = 255                       # down row 6: all 255
    s[dn + 7 * (I // 32):dn + 8 * (I // 32)] = 240 + np.arange(I // 32) % 16   # down row 7: base 240, deltas 0..15
    return w, c, s


def upload(w, c, s):
    desc = sd.desc_for(w)
    cb, sb = moe.packed_bytes(desc)
    codes = torch.empty(cb, dtype=torch.uint8, device=DEV)
    scales = torch.empty(sb, dtype=torch.uint8, device=DEV)
    moe.moe_mxfp4_pack(desc, torch.from_numpy(c).to(DEV), torch.from_numpy(s).to(DEV), 0, w.E, codes, scales)
    enc = moe.encode_scale4_layer(desc, scales)
    assert enc is not None
    desc4, scale4 = enc
    assert scale4.numel() == w.E * (2 * w.I + w.H + 3 * w.H * w.I // 64)
    return desc, codes, scales, desc4, scale4


def test_scale4_dequant_bitexact_and_byte_count():
    w, c, s = layer_with_extreme_rows(512, 256, 4, 2, 9000)
    desc, codes, scales, desc4, scale4 = upload(w, c, s)
    for e in range(w.E):
        for m, (rows, cols) in enumerate([(w.I, w.H), (w.I, w.H), (w.H, w.I)]):
            for fn in (moe.moe_mxfp4_dequant, moe.moe_mxfp4_dequant_bf16):
                a = torch.empty(rows, cols, dtype=torch.float32, device=DEV)
                b = torch.empty(rows, cols, dtype=torch.float32, device=DEV)
                fn(desc, codes, scales, e, m, a)
                fn(desc4, codes, scale4, e, m, b)
                torch.cuda.synchronize()
                assert np.array_equal(P.bits(a.cpu().numpy()), P.bits(b.cpu().numpy())), (e, m, fn.__name__)
    # the exports through scale4 also equal the oracle on the 8-bit table
    mc, ms = w.I * w.H // 2, w.I * w.H // 32
    out = torch.empty(w.H, w.I, dtype=torch.float32, device=DEV)
    moe.moe_mxfp4_dequant(desc4, codes, scale4, 1, 2, out)
    torch.cuda.synchronize()
    ce, se = w.code_bytes_per_expert, w.scale_bytes_per_expert
    ref = oracle.dequant(c[ce + 2 * mc:2 * ce], s[se + 2 * ms:2 * se], w.H, w.I)
    assert np.array_equal(P.bits(out.cpu().numpy()), P.bits(ref))
    # the K3 shape saves 505,856 of 17,547,264 bytes per expert (2.88%)
    d8 = moe.LayerDesc.make(7168, 1536, 896, 16)
    d4 = moe.LayerDesc.make(7168, 1536, 896, 16, moe.MOE_LAYOUT_SCALE4_V1)
    (c8, s8), (c4, s4) = moe.packed_bytes(d8), moe.packed_bytes(d4)
    assert c8 == c4 and (s8 - s4) // 896 == 505856


def test_scale4_reports_rows_it_cannot_code():
    w = synth.Workload("s4e", 81, 1, 256, 128, 3, 2, "bf16", weight_seed=9100)
    c, s = synth.experts(w)
    s = s.copy()
    s[w.scale_bytes_per_expert + 3] = 140          # expert 1, gate row 0: scales 119..123 and 140
    desc = sd.desc_for(w)
    cb, sb = moe.packed_bytes(desc)
    codes = torch.empty(cb, dtype=torch.uint8, device=DEV)
    scales = torch.empty(sb, dtype=torch.uint8, device=DEV)
    moe.moe_mxfp4_pack(desc, torch.from_numpy(c).to(DEV), torch.from_numpy(s).to(DEV), 0, w.E, codes, scales)
    assert moe.encode_scale4_layer(desc, scales) is None
    desc4 = moe.LayerDesc.make(w.H, w.I, w.E, w.k, moe.MOE_LAYOUT_SCALE4_V1)
    esc = torch.zeros(1, dtype=torch.int32, device=DEV)
    buf = torch.empty(moe.packed_bytes(desc4)[1], dtype=torch.uint8, device=DEV)
    moe.moe_mxfp4_scale4_encode(desc4, scales, 0, w.E, buf, esc)
    torch.cuda.synchronize()
    assert int(esc.item()) == 1


@pytest.mark.parametrize("T,xd", [(1, "bf16"), (3, "f32"), (1, "f32")])
def test_scale4_forward_and_stages_bit_identical(T, xd):
    w, c, s = layer_with_extreme_rows(512, 256, 6, 2, 9200)
    w = synth.Workload("s4", 80, T, 512, 256, 6, 2, xd, weight_seed=9200)
    desc, codes, scales, desc4, scale4 = upload(w, c, s)
    x = sd.tokens(w, range(T))
    wr = sd.router_w(w)
    outs = []
    for d, sc in ((desc, scales), (desc4, scale4)):
        out = torch.empty(T, w.H, dtype=torch.float32, device=DEV)
        idx = torch.empty(T, w.k, dtype=torch.int32, device=DEV)
        ws = torch.empty(moe.workspace_bytes(d, T, w.k), dtype=torch.uint8, device=DEV)
        moe.moe_mxfp4_forward(d, x, wr, None, codes, sc, w.k, out, ws, None, idx)
        h = torch.empty(T * w.k, w.I, dtype=torch.float32, device=DEV)
        moe.moe_mxfp4_gate_up(d, x, idx.reshape(-1), w.k, codes, sc, h)
        y = torch.empty(T * w.k, w.H, dtype=torch.float32, device=DEV)
        moe.moe_mxfp4_down(d, h, idx.reshape(-1), codes, sc, y)
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy() for t in (out, idx, h, y)])
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("xd", ["bf16", "f32"])
def test_scale4_split_k_stages_bit_identical(xd):
    """H and I multiples of 1024 (the K-split GEMVs of the model's width, which
    stage the scale4 deltas and bases in LDS): the routes-given and selecting
    gate/up stages and the down stage over every expert, extreme rows
    included, and the forward, equal the 8-bit table's bits.  The forward
    runs one bf16 token (more would take the 8-bit layer's grouped form) or
    three fp32 tokens (the decode form on both)."""
    H, I, E, k, T = 2048, 1024, 6, 2, 3
    _, c, s = layer_with_extreme_rows(H, I, E, k, 9250)
    w = synth.Workload("s4k", 83, T, H, I, E, k, xd, weight_seed=9250)
    desc, codes, scales, desc4, scale4 = upload(w, c, s)
    x = sd.tokens(w, range(T))
    pe = torch.arange(T * k, dtype=torch.int32, device=DEV) % E        # every expert, expert 1 included
    lg = torch.from_numpy(np.random.default_rng(4).standard_normal((T, E)).astype(np.float32)).to(DEV)
    wr = sd.router_w(w)
    outs = []
    for d, sc in ((desc, scales), (desc4, scale4)):
        h = torch.empty(T * k, I, dtype=torch.float32, device=DEV)
        moe.moe_mxfp4_gate_up(d, x, pe, k, codes, sc, h)
        y = torch.empty(T * k, H, dtype=torch.float32, device=DEV)
        moe.moe_mxfp4_down(d, h, pe, codes, sc, y)
        hs = torch.empty(T * k, I, dtype=torch.float32, device=DEV)
        idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
        wt = torch.empty(T, k, dtype=torch.float32, device=DEV)
        moe.moe_mxfp4_gate_up_select(d, x, lg, k, codes, sc, idx, wt, hs)
        tf = T if xd == "f32" else 1
        out = torch.empty(tf, H, dtype=torch.float32, device=DEV)
        ws = torch.empty(moe.workspace_bytes(d, tf, k), dtype=torch.uint8, device=DEV)
        moe.moe_mxfp4_forward(d, x[:tf], wr, None, codes, sc, k, out, ws)
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy() for t in (h, y, hs, idx, out)])
    assert not np.all(np.isfinite(outs[0][1]))  # the extreme down rows reach y
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_scale4_stack_bit_identical():
    """A two-layer stack (RMSNorm inside the router kernel, fp32 residual,
    fp32 activations into the K-split GEMVs) on scale4 side-cars equals the
    stack on the 8-bit tables bit for bit, one token and three."""
    H, I, E, k = 2048, 1024, 8, 2
    for T in (1, 3):
        w = synth.Workload("s4s", 84, T, H, I, E, k, "bf16", weight_seed=9260)
        layers8, layers4 = [], []
        for l in range(2):
            c, s = synth.experts(w, l)
            desc, codes, scales, desc4, scale4 = upload(w, c, s)
            layers8.append((codes, scales))
            layers4.append((codes, scale4))
        wrs = [sd.router_w(w, l) for l in range(2)]
        gam = [sd.gamma(w, l) for l in range(2)]
        x = sd.tokens(w, range(T))
        res = []
        for d, layers in ((desc, layers8), (desc4, layers4)):
            resid = torch.empty(T, H, dtype=torch.float32, device=DEV)
            ws = torch.empty(moe.stack_workspace_bytes(d, T, k), dtype=torch.uint8, device=DEV)
            moe.moe_mxfp4_stack_forward(d, [a for a, _ in layers], [b for _, b in layers], wrs, None, gam, w.eps, x, k,
                                        resid, ws)
            torch.cuda.synchronize()
            res.append(resid.cpu().numpy())
        assert np.all(np.isfinite(res[0]))
        assert np.array_equal(P.bits(res[0]), P.bits(res[1])), T


def test_scale4_many_bf16_tokens_decode_form_matches_oracle():
    H, I, E, k, T = 512, 256, 8, 2, 40
    w = synth.Workload("s4m", 82, T, H, I, E, k, "bf16", weight_seed=9300)
    c, s = synth.experts(w)
    ce, se = w.code_bytes_per_expert, w.scale_bytes_per_expert
    ex = [(c[e * ce:(e + 1) * ce], s[e * se:(e + 1) * se]) for e in range(E)]
    desc, codes, scales, desc4, scale4 = upload(w, c, s)
    x = sd.tokens(w, range(T))
    wr = sd.router_w(w)
    out = torch.empty(T, H, dtype=torch.float32, device=DEV)
    lg = torch.empty(T, E, dtype=torch.float32, device=DEV)
    idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    wt = torch.empty(T, k, dtype=torch.float32, device=DEV)
    ws = torch.empty(moe.workspace_bytes(desc4, T, k), dtype=torch.uint8, device=DEV)
    moe.moe_mxfp4_forward(desc4, x, wr, None, codes, scale4, k, out, ws, lg, idx, wt)
    torch.cuda.synchronize()
    xf = synth.tokens_f32(w, range(T))
    r_out, _, r_idx, r_w = oracle.moe_forward(xf, wr.cpu().numpy(), ex, H, I, k, logits_override=lg.cpu().numpy())
    assert np.array_equal(idx.cpu().numpy(), r_idx)
    P.assert_layer_close(out.cpu().numpy(), r_out, xf, r_idx, r_w, ex, H, I, E)


def test_scale4_model_shape_decode_bit_identical():
    w = synth.WORKLOADS["decode"]
    desc = sd.desc_for(w)
    codes, scales = sd.upload_layer(w, 0)
    desc4, scale4 = moe.encode_scale4_layer(desc, scales)
    wr = sd.router_w(w)
    for t in (0, 7):
        x = sd.tokens(w, [t])
        res = []
        for d, sc in ((desc, scales), (desc4, scale4)):
            out = torch.empty(1, w.H, dtype=torch.float32, device=DEV)
            ws = torch.empty(moe.workspace_bytes(d, 1, w.k), dtype=torch.uint8, device=DEV)
            moe.moe_mxfp4_forward(d, x, wr, None, codes, sc, w.k, out, ws)
            torch.cuda.synchronize()
            res.append(out.cpu().numpy())
        assert np.array_equal(P.bits(res[0]), P.bits(res[1])), t
    del codes, scales, scale4
    torch.cuda.empty_cache()
