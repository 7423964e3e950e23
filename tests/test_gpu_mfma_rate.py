"""The matrix-core rate entry (moe_mfma_rate), a measurement aid behind the
prefill form's ceiling: it runs every MFMA kind and writes every slot."""
import numpy as np
import pytest
import torch

import mxfp4_routed_expert_fp32_amd as moe

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.gpu
def test_mfma_rate_runs_every_kind():
    """The matrix-core rate entry (a measurement aid) runs each MFMA kind and
    writes every thread's sum: zero operands give exactly 0; random operands
    overwrite a sentinel in every slot (NaN included, which also differs)."""
    n_wg = 3
    sink = torch.empty(n_wg * 512, dtype=torch.float32, device=DEV)
    zeros = torch.zeros(65536, dtype=torch.uint8, device=DEV)
    rnd = torch.from_numpy(np.random.default_rng(5).integers(0, 256, 65536, dtype=np.uint8)).to(DEV)
    for kind in moe.MFMA_RATE_KINDS:
        sink.fill_(7.0)
        moe.moe_mfma_rate(kind, zeros, n_wg, 5, sink)
        torch.cuda.synchronize()
        assert torch.equal(sink, torch.zeros_like(sink)), kind
        sink.fill_(7.0)
        moe.moe_mfma_rate(kind, rnd, n_wg, 5, sink)
        torch.cuda.synchronize()
        assert not bool((sink == 7.0).any()), kind
