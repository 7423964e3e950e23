"""moe_mxfp4_forward_noalloc (the forward with its workspace in the library's
static device scratch) against moe_mxfp4_forward with a caller workspace, on
the same inputs: two calls in a row, the second with fewer tokens, at the
model shape (the prefill form for 64 bf16 tokens, then one decode token) and
on a small layer with fp32 activations; and the refusal of a call that needs
more than the 64 MiB scratch."""
import numpy as np
import pytest
import torch

import synth
import synth.device as sd
import mxfp4_routed_expert_fp32_amd as moe
from tests import _parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda"
SCRATCH_BYTES = 64 << 20


def both(desc, x, wr, bias, codes, scales, k, E, H):
    T = x.shape[0]
    res = []
    for noalloc in (True, False):
        out = torch.full((T, H), 5.0, dtype=torch.float32, device=DEV)
        logits = torch.empty(T, E, dtype=torch.float32, device=DEV)
        idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
        wt = torch.empty(T, k, dtype=torch.float32, device=DEV)
        if noalloc:
            moe.moe_mxfp4_forward_noalloc(desc, x, wr, bias, codes, scales, k, out, logits, idx, wt)
        else:
            ws = torch.empty(moe.workspace_bytes(desc, T, k), dtype=torch.uint8, device=DEV)
            moe.moe_mxfp4_forward(desc, x, wr, bias, codes, scales, k, out, ws, logits, idx, wt)
        torch.cuda.synchronize()
        res.append([t.cpu().numpy() for t in (out, logits, idx, wt)])
    return res


def assert_same(a, b):
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))


def test_noalloc_equals_forward_model_shape():
    w = synth.WORKLOADS["decode64_zipf"]
    desc = sd.desc_for(w)
    codes, scales = sd.upload_layer(w, 0)
    wr = sd.router_w(w)
    bias = sd.router_bias(w)
    x = sd.tokens(w, range(w.T))
    assert moe.workspace_bytes(desc, w.T, w.k) <= SCRATCH_BYTES
    a, b = both(desc, x, wr, bias, codes, scales, w.k, w.E, w.H)       # 64 tokens: prefill form
    assert_same(a, b)
    a, b = both(desc, x[5:6].contiguous(), wr, None, codes, scales, w.k, w.E, w.H)   # then one token
    assert_same(a, b)
    # a call whose workspace exceeds the scratch is refused before any launch
    T = 128
    assert moe.workspace_bytes(desc, T, w.k) > SCRATCH_BYTES
    xb = sd.tokens(w, range(T))
    out = torch.full((T, w.H), 5.0, dtype=torch.float32, device=DEV)
    with pytest.raises(moe.MoeError) as e:
        moe.moe_mxfp4_forward_noalloc(desc, xb, wr, bias, codes, scales, w.k, out)
    assert e.value.status == -12
    torch.cuda.synchronize()
    assert bool((out == 5.0).all())
    del codes, scales
    torch.cuda.empty_cache()


def test_noalloc_equals_forward_small_fp32():
    w = synth.Workload("na", 73, 9, 512, 256, 16, 4, "f32", weight_seed=8400)
    desc = sd.desc_for(w)
    codes, scales = sd.upload_layer(w, 0)
    wr = sd.router_w(w)
    x = sd.tokens(w, range(w.T))
    a, b = both(desc, x, wr, None, codes, scales, w.k, w.E, w.H)       # 9 fp32 tokens
    assert_same(a, b)
    a, b = both(desc, x[:2].contiguous(), wr, None, codes, scales, w.k, w.E, w.H)    # then 2
    assert_same(a, b)
    assert np.all(np.isfinite(a[0]))
