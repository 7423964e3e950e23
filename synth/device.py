"""Upload synthetic workload tensors to the GPU (tests and benchmark).

Generation happens on the host (synth.c); device copies go through torch, and
the weights enter the layer's device buffers through the library's own pack
entry point (moe_mxfp4_pack), so the tests exercise it on every upload.
"""
from __future__ import annotations

import numpy as np
import torch

import synth
import mxfp4_routed_expert_fp32_amd as moe


def desc_for(w: synth.Workload) -> moe.LayerDesc:
    return moe.LayerDesc.make(w.H, w.I, w.E, w.k)


def upload_layer(w: synth.Workload, layer: int = 0, device="cuda", chunk_experts: int = 64):
    """All E experts of one layer, generated in chunks into pinned host memory,
    copied to a device staging buffer and packed into the layer buffers."""
    desc = desc_for(w)
    cbytes, sbytes = moe.packed_bytes(desc)
    codes = torch.empty(cbytes, dtype=torch.uint8, device=device)
    scales = torch.empty(sbytes, dtype=torch.uint8, device=device)
    ce, se = w.code_bytes_per_expert, w.scale_bytes_per_expert
    n = min(chunk_experts, w.E)
    host_c = torch.empty(n * ce, dtype=torch.uint8, pin_memory=True)
    host_s = torch.empty(n * se, dtype=torch.uint8, pin_memory=True)
    dev_c = torch.empty(n * ce, dtype=torch.uint8, device=device)
    dev_s = torch.empty(n * se, dtype=torch.uint8, device=device)
    stream = torch.cuda.current_stream()
    for e0 in range(0, w.E, n):
        cnt = min(n, w.E - e0)
        stream.synchronize()  # staging buffers are free again
        synth.experts_into(w, layer, e0, cnt, host_c.data_ptr(), host_s.data_ptr())
        dev_c[:cnt * ce].copy_(host_c[:cnt * ce], non_blocking=True)
        dev_s[:cnt * se].copy_(host_s[:cnt * se], non_blocking=True)
        moe.moe_mxfp4_pack(desc, dev_c, dev_s, e0, cnt, codes, scales)
    stream.synchronize()
    del dev_c, dev_s
    return codes, scales


def router_w(w: synth.Workload, layer: int = 0, device="cuda") -> torch.Tensor:
    return torch.from_numpy(synth.router_w(w, layer)).to(device)


def router_bias(w: synth.Workload, layer: int = 0, device="cuda"):
    b = synth.router_bias(w, layer)
    return None if b is None else torch.from_numpy(b).to(device)


def tokens(w: synth.Workload, token_ids, device="cuda") -> torch.Tensor:
    """[T, H] activations in the workload's dtype (bf16 bit-exact with synth)."""
    if w.x_dtype == "bf16":
        bits = synth.tokens_bf16_bits(w, token_ids)
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(synth.tokens_f32(w, token_ids)).to(device)


def gamma(w: synth.Workload, layer: int, device="cuda") -> torch.Tensor:
    return torch.from_numpy(synth.gamma(w, layer)).to(device)
