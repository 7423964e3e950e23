"""Packed-int8 rows with fp16 row scales (the resident-spine GEMV on the
streaming skeleton): the fused dequant export bit for bit against the oracle,
and the GEMV against the oracle on both readings of the 2e-5 bar, at the
pages' 12288 x 7168 shape and at ragged shapes (rows not a multiple of a
workgroup's rows, a partial last wave), for 1-4 tokens of fp32 or bf16
activations."""
import numpy as np
import pytest
import torch

import oracle
import synth
import mxfp4_routed_expert_fp32_amd as moe
from tests import _parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda"


def dev_rows(q, s):
    return torch.from_numpy(q).to(DEV), torch.from_numpy(s.view(np.int16)).to(DEV)


def test_int8_dequant_bitexact():
    q, s = synth.int8_rows(31, 300, 1040)
    s = s.copy()
    s[0] = np.float16(6.0e-8).view(np.uint16)      # subnormal scale
    s[1] = np.float16(-0.5).view(np.uint16)        # negative scale
    s[2] = np.float16(65504.0).view(np.uint16)     # largest finite
    qd, sd_ = dev_rows(q, s)
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    moe.moe_int8_dequant(qd, sd_, out)
    torch.cuda.synchronize()
    assert np.array_equal(P.bits(out.cpu().numpy()), P.bits(oracle.int8_dequant(q, s)))


@pytest.mark.parametrize("N,K,T,xd,rpw", [(12288, 7168, 1, "f32", 0), (12288, 7168, 4, "f32", 0),
                                          (12288, 7168, 2, "bf16", 0), (1000, 1040, 3, "f32", 0),
                                          (77, 16, 1, "f32", 8), (4099, 16384, 1, "bf16", 8),
                                          (12288, 7168, 1, "f32", 48)])
def test_int8_gemv_matches_oracle(N, K, T, xd, rpw):
    q, s = synth.int8_rows(N + K, N, K)
    x = synth.normal_f32(synth.key(5, 0, 1, N + T), T * K).reshape(T, K)
    if xd == "bf16":
        bitsx = synth.f32_to_bf16_bits(x)
        x = synth.bf16_bits_to_f32(bitsx)
        xt = torch.from_numpy(bitsx.view(np.int16)).view(torch.bfloat16).to(DEV)
    else:
        xt = torch.from_numpy(x).to(DEV)
    qd, sd_ = dev_rows(q, s)
    y = torch.empty(T, N, dtype=torch.float32, device=DEV)
    moe.moe_int8_gemv(qd, sd_, xt, y, rows_per_workgroup=rpw)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    ref = oracle.int8_gemv(q, s, x)
    W = oracle.int8_dequant(q, s).astype(np.float64)
    A = np.abs(x).astype(np.float64) @ np.abs(W).T
    P.assert_out_close(got, ref)
    P.assert_elementwise(got, ref, A)

