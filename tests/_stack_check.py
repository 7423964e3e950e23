"""Layer-by-layer check of the MoE layer stack against the oracle (shared by
the stack tests and the benchmark's refusal gate).  Test infrastructure: it
calls the oracle."""
import numpy as np
import torch

import oracle
import synth
import mxfp4_routed_expert_fp32_amd as moe
from tests import _parity as P

DEV = "cuda"


def stack_layer_by_layer(w, desc, layers, gam, x, T, eps, k):
    """Runs the stack on the GPU with 1, 2, ..., L layers and checks layer l
    against the oracle started from the GPU's own residual after layer l - 1:
    the oracle normalises it, takes the GPU's router logits of those rows for
    selection (moe_rmsnorm + moe_router_logits give the stack kernel's bits),
    runs the layer and adds the residual.  Returns the worst (normwise,
    elementwise) errors, the GPU residual after the last layer, and the GPU
    residual entering each layer (its input before the norm)."""
    L = len(layers)
    ws = torch.empty(moe.stack_workspace_bytes(desc, T, k), dtype=torch.uint8, device=DEV)
    resid = torch.empty(T, w.H, dtype=torch.float32, device=DEV)
    if x.dtype == torch.bfloat16:    # the stack starts from x widened exactly
        r_prev = synth.bf16_bits_to_f32(x.view(torch.int16).cpu().numpy().view(np.uint16))
    else:
        r_prev = x.cpu().numpy()
    worst = (0.0, 0.0)
    inputs = []
    for l in range(L):
        inputs.append(r_prev)
        moe.moe_mxfp4_stack_forward(desc, [a[0] for a in layers[:l + 1]], [a[1] for a in layers[:l + 1]],
                                    [a[2] for a in layers[:l + 1]], None, gam[:l + 1], eps, x, k, resid, ws)
        torch.cuda.synchronize()
        r_gpu = resid.cpu().numpy().copy()
        n = oracle.rmsnorm(r_prev, gam[l].cpu().numpy(), eps)
        rp = torch.from_numpy(r_prev).to(DEV)
        nd = torch.empty_like(rp)
        moe.moe_rmsnorm(rp, gam[l], eps, nd)
        lg = torch.empty(T, w.E, dtype=torch.float32, device=DEV)
        moe.moe_router_logits(desc, nd, layers[l][2], None, lg)
        torch.cuda.synchronize()
        lg = lg.cpu().numpy()
        sel = np.unique(oracle.topk(lg, k))
        ex = {int(e): synth.expert(w, int(e), l) for e in sel}
        o, _, r_idx, r_w = oracle.moe_forward(n, layers[l][2].cpu().numpy(), ex, w.H, w.I, k, logits_override=lg)
        r_ref = oracle.residual_add(r_prev, o)
        nw = P.assert_out_close(r_gpu, r_ref)
        # the residual add rounds once on each side, on the same r_prev
        A = oracle.moe_abs_scale(n, r_idx, r_w, ex, w.H, w.I, w.E) + 2.0 ** -23 * np.abs(r_ref) / P.OUT_TOL
        ew = P.assert_elementwise(r_gpu, r_ref, A)
        worst = (max(worst[0], nw), max(worst[1], ew))
        r_prev = r_gpu
    return worst, r_prev, inputs
