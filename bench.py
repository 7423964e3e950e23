"""Benchmark of the routed MXFP4 MoE layer on one MI355X.

Default workload (`--workload decode`): single-token decode of one K3-shape
layer (H=7168, I=1536, E=896, top-16, bf16 activations, every expert resident
in HBM).  A step is one moe_mxfp4_forward call for one token: router logits,
top-k + softmax, expert gate/up + SwiGLU, expert down, rank-ordered combine.
Steps rotate over a pool of 256 distinct seeded tokens so that consecutive
steps route to different experts and the 256 MB last-level cache cannot serve
a replayed expert set.

Other workloads (same layer shape): `decode64_zipf` (64 tokens per step,
Zipf(1.1) router bias), `prefill4096` (4096 tokens per step, uniform routing),
`stack12` (12 layers with RMSNorm + residual, one token per step, replayed
as a HIP graph).

Prints one JSON line.  The roofline object describes the dominant kernel
(decode: the gate/up GEMV, timed over a run of back-to-back launches with
HIP events on the stream it runs on); `cpu_baseline` times the CPU oracle on the host cores on a
bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
MXFP4_PEAK_TFLOPS = 10100.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None)
    p.add_argument("--warmup", type=int, default=None)
    p.add_argument("--workload", default="decode", choices=["decode", "decode64_zipf", "prefill4096", "stack12"])
    p.add_argument("--pool", type=int, default=256)
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    return p.parse_args()


DEFAULT_STEPS = {"decode": (400, 40), "decode64_zipf": (100, 10), "prefill4096": (20, 3), "stack12": (100, 10)}

# Source files each dominant kernel is built from: HBM traffic measured with
# rocprofv3 counters is reported only while these files still hash to the
# value recorded next to the counters.
KERNEL_SOURCES = {
    "k_gateup_gemv": ["expert_gemv.hip", "common.h", "topk.h"],
    "k_gateup_mfma": ["expert_mfma.hip", "common.h"],
}


def source_hash(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "mxfp4_routed_expert_fp32_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch from profiles/hbm_traffic_<kernel>_<workload>.txt
    (FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by its reading for a
    copy kernel of known size), or None when that file is missing or the
    kernel's sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_%s_%s.txt" % (kernel, workload))
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            kv[key.strip()] = val.strip()
    if kv.get("source_sha256") != source_hash(kernel):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    a = parse()
    if a.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % a.gpus, file=sys.stderr)
        sys.exit(2)
    steps, warmup = DEFAULT_STEPS[a.workload]
    a.steps = steps if a.steps is None else a.steps
    a.warmup = warmup if a.warmup is None else a.warmup
    if a.workload == "decode":
        res = bench_decode(a)
    elif a.workload in ("decode64_zipf", "prefill4096"):
        res = bench_batch(a)
    else:
        res = bench_stack(a)
    print(json.dumps(res), flush=True)


def common_fields(a, metric, value, unit, ms_step, config, roofline):
    return {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
            "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "f32 accumulate; bf16 activations; mxfp4 weights", "data": "synthetic (seeded)",
            "config": config, "roofline": roofline, "cpu_baseline": None}


def hold_queue(seconds):
    """Keep the GPU busy on the current stream for about `seconds` (a bounded
    spin kernel) so that the launches enqueued next run back to back: two
    events around a run of launches then time the kernels (and the launch
    gaps between them), not the host's enqueue gaps."""
    import torch
    torch.cuda._sleep(int(seconds * 2.4e9))


def hold_for(n, enqueue_s, kernel_s):
    """Hold the queue just long enough that the host, enqueuing n launches at
    enqueue_s each, stays ahead of the GPU running them at kernel_s each (both
    measured on the warm-up launches), plus 0.5 ms.  A long hold is
    measurably wrong: after a 40 ms spin of one wave, 32-us GEMV launches ran
    about 7% slower than the same launches back to back (the clock ramps back
    up), and a 6 ms spin still cost about 4%."""
    hold_queue(min(1.5 * n * max(0.0, enqueue_s - kernel_s) + 0.5e-3, 0.02))


def warm(launch, n):
    """Runs n warm-up launches; returns (host seconds per enqueue, GPU seconds per launch)."""
    import torch
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    t0 = time.perf_counter()
    for i in range(n):
        launch(i)
    host = (time.perf_counter() - t0) / n
    e1.record()
    torch.cuda.synchronize()
    return host, e0.elapsed_time(e1) * 1e-3 / n


def timed(step, n, warmup):
    import torch
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(n):
        step(warmup + i)
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / n


# --------------------------------------------------------------------------- decode

def bench_decode(a):
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

    parity = parity_gate(w, step, out, logits, idx, wr, lambda t: synth.tokens_f32(w, [t]), [0, 1])

    # routes of every pool token (for the stage timing below)
    routes = torch.empty(a.pool, k, dtype=torch.int32, device=dev)
    for i in range(a.pool):
        step(i)
        routes[i].copy_(idx[0])
    torch.cuda.synchronize()

    ms_step = timed(step, a.steps, a.warmup)

    # dominant kernel: gate/up + SwiGLU GEMV, timed over back-to-back launches on the
    # stream it runs on, with the same routes and tokens as the steps above
    hbuf = torch.empty(k, I, dtype=torch.float32, device=dev)
    enqueue_s, kernel_s = warm(
        lambda i: moe.moe_mxfp4_gate_up(desc, pool[i % a.pool:i % a.pool + 1], routes[i % a.pool], k, codes,
                                        scales, hbuf), max(1, a.warmup))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    hold_for(a.steps, enqueue_s, kernel_s)
    e0.record()
    for i in range(a.steps):
        j = (a.warmup + i) % a.pool
        moe.moe_mxfp4_gate_up(desc, pool[j:j + 1], routes[j], k, codes, scales, hbuf)
    e1.record()
    torch.cuda.synchronize()
    gu_ms = e0.elapsed_time(e1) / a.steps
    gu_bytes = k * 2 * (I * H // 2 + I * H // 32) + H * 2 + k * I * 4
    achieved = gu_bytes / (gu_ms * 1e-3) / 1e9

    expert_bytes = k * w.expert_bytes
    layer_bytes = expert_bytes + E * H * 4 + H * 2 + H * 4
    res = common_fields(
        a, "MoE-layer decode tokens/s (one token per step, one K3-shape layer)", 1.0 / (ms_step * 1e-3),
        "tokens/s", ms_step,
        {"workload": "decode: T=1, H=7168, I=1536, E=896, k=16, bf16 x, all experts resident, "
                     "256-token rotating pool",
         "global_batch": 1, "layer_bytes_per_token": layer_bytes,
         "layer_GBps": layer_bytes / (ms_step * 1e-3) / 1e9, "expert_bytes_per_token": expert_bytes,
         "parity_max_err": parity},
        {"bound": "hbm", "kernel": "k_gateup_gemv (routes given)", "achieved": achieved, "peak": HBM_PEAK_GBS,
         "unit": "GB/s",
         "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic("k_gateup_gemv", "decode"),
         "avg_launch_us": gu_ms * 1e3, "bytes_per_launch": gu_bytes})
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, a.cpu_seconds, 1)
    return res


# --------------------------------------------------------------------------- batched decode / prefill

def bench_batch(a):
    import numpy as np
    import torch

    import synth
    import synth.device as sd
    import mxfp4_routed_expert_fp32_amd as moe

    w = synth.WORKLOADS[a.workload]
    desc = sd.desc_for(w)
    dev = "cuda"
    T, k, H, I, E = w.T, w.k, w.H, w.I, w.E
    t0 = time.time()
    codes, scales = sd.upload_layer(w, 0)
    wr = sd.router_w(w)
    bias = sd.router_bias(w)
    nbatch = 8 if T <= 64 else 2                 # rotating batches of distinct tokens
    xs = [sd.tokens(w, range(b * T, (b + 1) * T)) for b in range(nbatch)]
    print("setup in %.1f s" % (time.time() - t0), file=sys.stderr, flush=True)
    out = torch.empty(T, H, dtype=torch.float32, device=dev)
    logits = torch.empty(T, E, dtype=torch.float32, device=dev)
    idx = torch.empty(T, k, dtype=torch.int32, device=dev)
    wt = torch.empty(T, k, dtype=torch.float32, device=dev)
    ws = torch.empty(moe.workspace_bytes(desc, T, k), dtype=torch.uint8, device=dev)

    def step(i):
        moe.moe_mxfp4_forward(desc, xs[i % nbatch], wr, bias, codes, scales, k, out, ws, logits, idx, wt)

    b_h = None if bias is None else bias.cpu().numpy()
    parity = parity_gate(w, step, out, logits, idx, wr, lambda t: synth.tokens_f32(w, range(T))[[t]], [0, T - 1],
                         bias=b_h, rows=True)
    unions, maxload = [], []
    for b in range(nbatch):
        step(b)
        torch.cuda.synchronize()
        ids = idx.cpu().numpy()
        unions.append(len(np.unique(ids)))
        maxload.append(int(np.bincount(ids.reshape(-1), minlength=E).max()))
    ms_step = timed(step, a.steps, a.warmup)
    union = float(np.mean(unions))
    touched = union * w.expert_bytes + E * H * 4 + T * H * 2 + T * H * 4
    gbps = touched / (ms_step * 1e-3) / 1e9
    flops = 2.0 * T * k * 3 * H * I + 2.0 * T * E * H
    tflops = flops / (ms_step * 1e-3) / 1e12
    cfg = {"workload": "%s: T=%d, H=%d, I=%d, E=%d, k=%d, bf16 x%s" % (
               a.workload, T, H, I, E, k, ", Zipf(1.1) router bias" if bias is not None else ", uniform routing"),
           "global_batch": T, "experts_touched_mean": union, "max_expert_load": max(maxload),
           "touched_bytes_per_step": touched, "layer_GBps": gbps, "algorithmic_TFLOPs": tflops,
           "frac_bf16_mfma_peak": tflops / BF16_PEAK_TFLOPS, "frac_mxfp4_mfma_peak": tflops / MXFP4_PEAK_TFLOPS,
           "parity_max_err": parity}
    # dominant kernel: the grouped gate/up GEMM (k_gateup_mfma), timed over a
    # run of back-to-back launches with HIP events on its stream, over the sorted
    # routes of each rotating batch
    P = T * k
    mb = moe.max_expert_blocks(E, P)
    nsw = moe.sort_workspace_bytes(E, T, k)
    sort_ws = torch.empty(nsw, dtype=torch.uint8, device=dev) if nsw else None
    stage = []
    for b in range(nbatch):
        step(b)
        offs = torch.empty(E + 1, dtype=torch.int32, device=dev)
        pairs = torch.empty(P, dtype=torch.int32, device=dev)
        moe.moe_sort_by_expert(idx, E, offs, pairs, sort_ws)
        blocks = torch.empty(mb, 4, dtype=torch.int32, device=dev)
        nb = torch.empty(1, dtype=torch.int32, device=dev)
        moe.moe_expert_blocks(offs, P, blocks, nb)
        stage.append((pairs, blocks, nb))
    hterm = torch.empty(2, P, I, dtype=torch.bfloat16, device=dev)

    def gate_up(i):
        j = i % nbatch
        moe.moe_mxfp4_grouped_gate_up(desc, xs[j], k, stage[j][0], stage[j][1], stage[j][2], codes, scales, hterm)

    enqueue_s, kernel_s = warm(gate_up, max(2, a.warmup))
    nl = max(a.steps, 2 * nbatch)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    hold_for(nl, enqueue_s, kernel_s)
    e0.record()
    for i in range(nl):
        gate_up(i)
    e1.record()
    torch.cuda.synchronize()
    gu_avg_ms = e0.elapsed_time(e1) / nl
    gu_ms = [gu_avg_ms] * nl
    gu_w = 2 * (I * H // 2 + I * H // 32)                     # gate + up bytes of one expert
    gu_bytes = [unions[i % nbatch] * gu_w + T * H * 2 + P * I * 4 for i in range(nl)]
    gu_flops = 4.0 * H * I * P
    cfg["gate_up_avg_launch_us"] = gu_avg_ms * 1e3
    if a.workload == "prefill4096":
        ach = gu_flops / (gu_avg_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": "k_gateup_mfma", "achieved": ach, "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": ach / BF16_PEAK_TFLOPS,
                "traffic": measured_traffic("k_gateup_mfma", a.workload), "avg_launch_us": gu_avg_ms * 1e3,
                "flops_per_launch": gu_flops, "frac_mxfp4_mfma_peak": ach / MXFP4_PEAK_TFLOPS,
                "weight_GBps": float(np.mean(gu_bytes)) / (gu_avg_ms * 1e-3) / 1e9}
    else:
        ach = float(np.sum(gu_bytes)) / (float(np.sum(gu_ms)) * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": "k_gateup_mfma", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": ach / HBM_PEAK_GBS, "traffic": measured_traffic("k_gateup_mfma", a.workload),
                "avg_launch_us": gu_avg_ms * 1e3, "bytes_per_launch": float(np.mean(gu_bytes))}
    res = common_fields(a, "MoE-layer tokens/s (%s)" % a.workload, T / (ms_step * 1e-3), "tokens/s", ms_step, cfg,
                        roof)
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, a.cpu_seconds, 1)
    return res


# --------------------------------------------------------------------------- stack

def bench_stack(a):
    import numpy as np
    import torch

    import synth
    import synth.device as sd
    import mxfp4_routed_expert_fp32_amd as moe

    w = synth.WORKLOADS["stack12"]
    desc = sd.desc_for(w)
    dev = "cuda"
    t0 = time.time()
    layers = [sd.upload_layer(w, l) for l in range(w.layers)]
    wrs = [sd.router_w(w, l) for l in range(w.layers)]
    gam = [sd.gamma(w, l) for l in range(w.layers)]
    print("setup: %d layers resident in %.1f s" % (w.layers, time.time() - t0), file=sys.stderr, flush=True)
    pool = sd.tokens(w, range(a.pool))
    x = torch.empty(1, w.H, dtype=torch.bfloat16, device=dev)
    resid = torch.empty(1, w.H, dtype=torch.float32, device=dev)
    ws = torch.empty(moe.stack_workspace_bytes(desc, 1, w.k), dtype=torch.uint8, device=dev)
    args = ([l[0] for l in layers], [l[1] for l in layers], wrs, None, gam, w.eps)
    graph = moe.StackGraph(desc, *args, x, w.k, resid, ws)

    def step(i):
        x.copy_(pool[i % a.pool:i % a.pool + 1])
        graph.launch()

    def eager(i):
        x.copy_(pool[i % a.pool:i % a.pool + 1])
        moe.moe_mxfp4_stack_forward(desc, *args, x, w.k, resid, ws)

    step(0)
    torch.cuda.synchronize()
    g0 = resid.cpu().numpy().copy()
    eager(0)
    torch.cuda.synchronize()
    assert np.array_equal(g0.view(np.uint32), resid.cpu().numpy().view(np.uint32)), "graph != eager"
    ms_graph = timed(step, a.steps, a.warmup)
    ms_eager = timed(eager, max(10, a.steps // 4), 3)
    per_tok = w.layers * (w.k * w.expert_bytes + w.E * w.H * 4)
    gbps = per_tok / (ms_graph * 1e-3) / 1e9
    cfg = {"workload": "stack12: 12 layers x (RMSNorm eps=1e-6 + MoE H=7168 I=1536 E=896 k=16 + residual), T=1, "
                       "hipGraph replay, 256-token rotating pool",
           "global_batch": 1, "bytes_per_token": per_tok, "GBps": gbps, "ms_per_token_eager": ms_eager,
           "graph_equals_eager": True}
    roof = {"bound": "hbm", "kernel": "stack", "achieved": gbps, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": gbps / HBM_PEAK_GBS, "traffic": None}
    graph.close()
    return common_fields(a, "12-layer MoE stack decode tokens/s", 1.0 / (ms_graph * 1e-3), "tokens/s", ms_graph,
                         cfg, roof)


# --------------------------------------------------------------------------- checks and CPU baseline

def parity_gate(w, step, out, logits, idx, wr, tokens_of, ts, bias=None, rows=False):
    """Refuse to report a number if the layer disagrees with the oracle (run on
    the GPU's logits) on sample tokens."""
    import numpy as np
    import torch

    import oracle
    import synth
    from tests import _parity as P

    worst = 0.0
    wr_h = wr.cpu().numpy()
    for t in ts:
        if rows:           # one batch holds every sample token: row t of step 0
            if t == ts[0]:
                step(0)
                torch.cuda.synchronize()
            r = t
        else:              # one token per step: step t, row 0
            step(t)
            torch.cuda.synchronize()
            r = 0
        lg_all, idx_all, out_all = logits.cpu().numpy(), idx.cpu().numpy(), out.cpu().numpy()
        lg = lg_all[r:r + 1]
        sel = np.unique(oracle.topk(lg, w.k))
        ex = {int(e): synth.expert(w, int(e)) for e in sel}
        r_out, _, r_idx, _ = oracle.moe_forward(tokens_of(t), wr_h, ex, w.H, w.I, w.k, bias=bias,
                                                logits_override=lg)
        if not np.array_equal(idx_all[r:r + 1], r_idx):
            raise SystemExit("parity gate failed: top-k differs from the oracle")
        err = float(P.normwise_err(out_all[r:r + 1], r_out).max())
        if not err <= P.OUT_TOL:
            raise SystemExit("parity gate failed: normwise error %g" % err)
        worst = max(worst, err)
    return worst


def cpu_baseline(w, seconds, tokens_per_call):
    """The oracle as it is, on the host cores, on whole tokens of the same
    workload until `seconds` of wall time have been spent (at least 2 tokens)."""
    import numpy as np

    import oracle
    import synth

    wr = synth.router_w(w)
    bias = synth.router_bias(w)
    cores = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        cores = min(cores, int(os.environ["OMP_NUM_THREADS"]))
    n, spent = 0, 0.0
    while n < 2 or spent < seconds:
        t = 100000 + n
        x = synth.tokens_f32(w, [t])
        sel = np.unique(oracle.topk(oracle.router_logits(x, wr, bias), w.k))
        ex = {int(e): synth.expert(w, int(e)) for e in sel}
        t0 = time.perf_counter()
        oracle.moe_forward(x, wr, ex, w.H, w.I, w.k, bias=bias, nthreads=cores)
        spent += time.perf_counter() - t0
        n += 1
        if n >= 512:
            break
    return {"value": n / spent, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "%d tokens of the %s workload, one oracle call each, %.1f s of oracle time" % (
                n, w.name, spent)}


if __name__ == "__main__":
    main()
