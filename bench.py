"""Benchmark of the routed MXFP4 MoE layer on one MI355X.

Default workload: single-token decode of one K3-shape layer (H=7168, I=1536,
E=896, top-16, bf16 activations, every expert resident in HBM).  A step is one
moe_mxfp4_forward call for one token: router logits, top-k + softmax, expert
gate/up + SwiGLU, expert down, rank-ordered combine.  Steps rotate over a pool
of 256 distinct seeded tokens so that consecutive steps route to different
experts and the 256 MB last-level cache cannot serve a replayed expert set.

Prints one JSON line (see the README of the measurement in the design doc).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=400)
    p.add_argument("--warmup", type=int, default=40)
    p.add_argument("--pool", type=int, default=256)
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    return p.parse_args()


def main():
    a = parse()
    if a.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % a.gpus, file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import synth
    import synth.device as sd
    import mxfp4_routed_expert_fp32_amd as moe

    w = synth.WORKLOADS["decode"]
    desc = sd.desc_for(w)
    dev = "cuda"
    t0 = time.time()
    codes, scales = sd.upload_layer(w, 0)
    wr = sd.router_w(w)
    pool = sd.tokens(w, range(a.pool))                      # [pool, H] bf16
    print("setup: layer resident (%.2f GB) in %.1f s" % ((codes.numel() + scales.numel()) / 1e9,
                                                          time.time() - t0), file=sys.stderr, flush=True)
    k, H, I, E = w.k, w.H, w.I, w.E
    out = torch.empty(1, H, dtype=torch.float32, device=dev)
    logits = torch.empty(1, E, dtype=torch.float32, device=dev)
    idx = torch.empty(1, k, dtype=torch.int32, device=dev)
    wt = torch.empty(1, k, dtype=torch.float32, device=dev)
    ws = torch.empty(moe.workspace_bytes(desc, 1, k), dtype=torch.uint8, device=dev)

    def step(i):
        x = pool[i % a.pool:i % a.pool + 1]
        moe.moe_mxfp4_forward(desc, x, wr, None, codes, scales, k, out, ws, logits, idx, wt)

    # ---- parity gate: refuse to report a number if the layer disagrees with the oracle
    parity = parity_gate(w, pool, wr, step, out, logits, idx)

    # ---- routes of every pool token (for the stage timing below)
    routes = torch.empty(a.pool, k, dtype=torch.int32, device=dev)
    for i in range(a.pool):
        step(i)
        routes[i].copy_(idx[0])
    torch.cuda.synchronize()

    # ---- timed region: whole layer
    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(a.steps):
        step(a.warmup + i)
    ev1.record()
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / a.steps

    # ---- dominant kernel: gate/up + SwiGLU GEMV, timed launch by launch on the
    # stream it runs on, with the same routes and tokens as the steps above
    hbuf = torch.empty(k, I, dtype=torch.float32, device=dev)
    for i in range(a.warmup):
        moe.moe_mxfp4_gate_up(desc, pool[i % a.pool:i % a.pool + 1], routes[i % a.pool], k, codes, scales, hbuf)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps)]
    for i in range(a.steps):
        j = (a.warmup + i) % a.pool
        starts[i].record()
        moe.moe_mxfp4_gate_up(desc, pool[j:j + 1], routes[j], k, codes, scales, hbuf)
        ends[i].record()
    torch.cuda.synchronize()
    gu_ms = float(np.mean([s.elapsed_time(e) for s, e in zip(starts, ends)]))
    gu_bytes = k * 2 * (I * H // 2 + I * H // 32) + H * 2 + k * I * 4
    achieved = gu_bytes / (gu_ms * 1e-3) / 1e9

    expert_bytes = k * w.expert_bytes
    layer_bytes = expert_bytes + E * H * 4 + H * 2 + H * 4
    res = {
        "metric": "MoE-layer decode tokens/s (one token per step, one K3-shape layer)",
        "value": 1.0 / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 accumulate; bf16 activations; mxfp4 weights",
        "data": "synthetic (seeded; 256-token rotating pool)",
        "config": {"workload": "decode: T=1, H=7168, I=1536, E=896, k=16, bf16 x, all experts resident",
                   "global_batch": 1, "layer_bytes_per_token": layer_bytes,
                   "layer_GBps": layer_bytes / (ms_step * 1e-3) / 1e9,
                   "expert_bytes_per_token": expert_bytes, "parity_max_err": parity},
        "roofline": {"bound": "hbm", "kernel": "k_gateup_gemv", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "avg_launch_us": gu_ms * 1e3, "bytes_per_launch": gu_bytes},
        "cpu_baseline": None,
    }
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, a.cpu_seconds)
    print(json.dumps(res), flush=True)


def parity_gate(w, pool, wr, step, out, logits, idx):
    import numpy as np
    import torch

    import oracle
    import synth
    from tests import _parity as P

    worst = 0.0
    wr_h = wr.cpu().numpy()
    for t in (0, 1):
        step(t)
        torch.cuda.synchronize()
        lg = logits.cpu().numpy()
        sel = np.unique(oracle.topk(lg, w.k))
        ex = {int(e): synth.expert(w, int(e)) for e in sel}
        r_out, _, r_idx, _ = oracle.moe_forward(synth.tokens_f32(w, [t]), wr_h, ex, w.H, w.I, w.k,
                                                logits_override=lg)
        if not np.array_equal(idx.cpu().numpy(), r_idx):
            raise SystemExit("parity gate failed: top-k differs from the oracle")
        err = float(P.normwise_err(out.cpu().numpy(), r_out).max())
        if not err <= P.OUT_TOL:
            raise SystemExit("parity gate failed: normwise error %g" % err)
        worst = max(worst, err)
    return worst


def cpu_baseline(w, seconds):
    """The oracle as it is, on the host cores, on whole tokens of the same
    workload until `seconds` of wall time have been spent (at least 2 tokens)."""
    import numpy as np

    import oracle
    import synth

    wr = synth.router_w(w)
    cores = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        cores = min(cores, int(os.environ["OMP_NUM_THREADS"]))
    n, spent = 0, 0.0
    while n < 2 or spent < seconds:
        t = 1000 + n
        x = synth.tokens_f32(w, [t])
        sel = np.unique(oracle.topk(oracle.router_logits(x, wr), w.k))
        ex = {int(e): synth.expert(w, int(e)) for e in sel}
        t0 = time.perf_counter()
        oracle.moe_forward(x, wr, ex, w.H, w.I, w.k, nthreads=cores)
        spent += time.perf_counter() - t0
        n += 1
        if n >= 64:
            break
    return {"value": n / spent, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "%d decode tokens (one layer each), %.1f s of oracle time" % (n, spent)}


if __name__ == "__main__":
    main()
