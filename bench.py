"""Benchmark of the routed MXFP4 MoE layer on one MI355X.

The default run (`--workload all`) measures the model-shape workloads in one
process and prints ONE JSON line.  Its top-level figures are single-token
decode of one K3-shape layer (H=7168, I=1536, E=896, top-16, bf16
activations, every expert resident in HBM); the others are sub-objects under
"workloads":
  - decode64_zipf: 64 tokens per step, Zipf(1.1) router bias;
  - prefill4096: 4096 tokens per step, uniform routing (grouped GEMMs on MFMA);
  - stack12: 12 layers with RMSNorm + residual, one token per step, replayed
    as a HIP graph (plus the next-layer route hint's accuracy);
  - decode_streamed: the decode workload with the experts in host memory and
    a device residency cache (host-link GB/s, pageable and pinned);
  - spine_int8: the packed-int8 resident-spine GEMV (12288 x 7168).
A step is one call of the layer (or of the stack graph).  Decode steps
rotate over a pool of 256 distinct seeded tokens and batch steps over
distinct token batches, so consecutive steps route to different experts and
the 256 MB last-level cache cannot serve a replayed expert set.

Every workload is gated on parity first: sample tokens are checked against
the CPU oracle (run on the GPU's own logits) on both readings of the output
bar, and no number is printed if they disagree.  Each workload's `roofline`
object describes the kernels its timed step runs: their algorithmic bytes
(or flops) per launch divided by their mean launch time, measured here with
HIP events over back-to-back launches on the stream they run on.  `traffic`
is the HBM bytes of the same kernels read from rocprofv3 counter summaries
under profiles/ (null when those kernels' sources changed since).
`cpu_baseline` times the oracle on the host cores on a bounded sample of the
decode workload.
"""
import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
MXFP4_PEAK_TFLOPS = 10100.0

WORKLOADS = ["decode", "decode64_zipf", "prefill4096", "stack12", "decode_streamed", "spine_int8"]
DEFAULT_STEPS = {"decode": (400, 40), "decode64_zipf": (100, 10), "prefill4096": (20, 3), "stack12": (100, 10),
                 "decode_streamed": (40, 0), "spine_int8": (200, 20)}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None, help="timed steps of the primary workload")
    p.add_argument("--warmup", type=int, default=None)
    p.add_argument("--workload", default="all", choices=["all"] + WORKLOADS)
    p.add_argument("--pool", type=int, default=256)
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    return p.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# --------------------------------------------------------------------------- counter traffic

# Source files each measured kernel is built from: HBM traffic measured with
# rocprofv3 counters is reported only while these files still hash to the
# value recorded next to the counters.
KERNEL_SOURCES = {
    "k_gateup_ks": ["expert_gemv.hip", "common.h", "topk.h"],
    "k_down_ks": ["expert_gemv.hip", "common.h"],
    "k_gateup_mfma": ["expert_mfma.hip", "common.h"],
    "k_down_mfma": ["expert_mfma.hip", "common.h"],
    "k_int8_gemv": ["int8_gemv.hip", "common.h"],
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


def sum_traffic(items):
    vals = [measured_traffic(k, w) for k, w in items]
    return None if any(v is None for v in vals) else float(sum(vals))


# --------------------------------------------------------------------------- timing

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


def kernel_us(launch, n, warmup):
    """Mean duration of one launch over n back-to-back launches (HIP events on
    the current stream, after a queue hold)."""
    import torch
    enqueue_s, kernel_s = warm(launch, max(2, warmup))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    hold_for(n, enqueue_s, kernel_s)
    e0.record()
    for i in range(n):
        launch(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n


def time_steps(step, n, warmup, groups=5):
    """Times exactly n steps after `warmup` untimed ones, between two events
    with a device synchronisation on both sides.  Events between equal groups
    of steps give the spread: median, min and max of the group means."""
    import torch
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    groups = max(1, min(groups, n))
    sizes = [n // groups + (1 if g < n % groups else 0) for g in range(groups)]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(groups + 1)]
    evs[0].record()
    i = 0
    for g, sz in enumerate(sizes):
        for _ in range(sz):
            step(warmup + i)
            i += 1
        evs[g + 1].record()
    torch.cuda.synchronize()
    ms = evs[0].elapsed_time(evs[-1]) / n
    per = [evs[g].elapsed_time(evs[g + 1]) / sizes[g] for g in range(groups)]
    return ms, {"median_ms": statistics.median(per), "min_ms": min(per), "max_ms": max(per),
                "groups": groups}


# --------------------------------------------------------------------------- parity gates

def refuse(msg):
    log("parity gate failed: " + msg)
    raise SystemExit("parity gate failed: " + msg)


def gate_tokens(w, xf, logits, idx, wt, out, wr_h, bias=None, layer=0):
    """Oracle on the GPU's logits for the given tokens; returns (normwise,
    elementwise) maxima or refuses."""
    import numpy as np

    import oracle
    import synth
    from tests import _parity as P

    sel = np.unique(oracle.topk(logits, w.k))
    ex = {int(e): synth.expert(w, int(e), layer) for e in sel}
    r_out, _, r_idx, r_w = oracle.moe_forward(xf, wr_h, ex, w.H, w.I, w.k, bias=bias, logits_override=logits)
    if not np.array_equal(idx, r_idx):
        refuse("top-k differs from the oracle")
    if P.weights_rel_err(wt, r_w) > 2 * (w.k + 4) * 2.0 ** -24:
        refuse("combine weights differ from the oracle")
    if not np.all(np.isfinite(out)):
        refuse("non-finite output")
    nw = float(P.normwise_err(out, r_out).max())
    A = oracle.moe_abs_scale(xf, r_idx, r_w, ex, w.H, w.I, w.E)
    ew = P.elementwise_ratio(out, r_out, A)
    if not (nw <= P.OUT_TOL and ew <= P.OUT_TOL):
        refuse("normwise %g, elementwise %g" % (nw, ew))
    return nw, ew


def parity_obj(tokens, nw, ew):
    return {"tokens_checked": tokens, "normwise_max": nw, "elementwise_max": ew, "tolerance": 2e-5,
            "readings": "normwise max|g-r|/max|r| per token; elementwise |g-r|/A with A the oracle's "
                        "magnitude scale"}


# --------------------------------------------------------------------------- shared state

class Ctx:
    """The model-shape layer 0 (shared by decode, the batch workloads and the
    stack's first layer) and its router."""

    def __init__(self):
        import synth
        import synth.device as sd
        t0 = time.time()
        w = synth.WORKLOADS["decode"]
        self.codes, self.scales = sd.upload_layer(w, 0)
        self.wr = sd.router_w(w)
        log("setup: layer 0 resident (%.2f GB) in %.1f s" % ((self.codes.numel() + self.scales.numel()) / 1e9,
                                                            time.time() - t0))


def base_fields(metric, value, unit, steps, warmup, ms_step, spread, config, roofline, parity):
    return {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": steps, "warmup": warmup,
            "ms_per_step": ms_step, "ms_per_step_spread": spread, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f32 accumulate; bf16 activations; mxfp4 weights",
            "data": "synthetic (seeded)", "config": config, "parity": parity, "roofline": roofline}


# --------------------------------------------------------------------------- decode

def bench_decode(a, ctx, steps, warmup):
    import numpy as np
    import torch

    import synth
    import synth.device as sd
    import mxfp4_routed_expert_fp32_amd as moe

    w = synth.WORKLOADS["decode"]
    desc = sd.desc_for(w)
    dev = "cuda"
    codes, scales, wr = ctx.codes, ctx.scales, ctx.wr
    pool = sd.tokens(w, range(a.pool))                      # [pool, H] bf16
    k, H, I, E = w.k, w.H, w.I, w.E
    out = torch.empty(1, H, dtype=torch.float32, device=dev)
    logits = torch.empty(1, E, dtype=torch.float32, device=dev)
    idx = torch.empty(1, k, dtype=torch.int32, device=dev)
    wt = torch.empty(1, k, dtype=torch.float32, device=dev)
    ws = torch.empty(moe.workspace_bytes(desc, 1, k), dtype=torch.uint8, device=dev)

    def step(i):
        x = pool[i % a.pool:i % a.pool + 1]
        moe.moe_mxfp4_forward(desc, x, wr, None, codes, scales, k, out, ws, logits, idx, wt)

    # parity gate on two tokens
    wr_h = wr.cpu().numpy()
    gate = (0.0, 0.0)
    for t in (0, 1):
        step(t)
        torch.cuda.synchronize()
        r = gate_tokens(w, synth.tokens_f32(w, [t]), logits.cpu().numpy(), idx.cpu().numpy(), wt.cpu().numpy(),
                        out.cpu().numpy(), wr_h)
        gate = (max(gate[0], r[0]), max(gate[1], r[1]))
    log("decode: parity ok (normwise %.3g, elementwise %.3g)" % gate)

    # logits and routes of every pool token (for the kernel timing below)
    logits_all = torch.empty(a.pool, E, dtype=torch.float32, device=dev)
    routes = torch.empty(a.pool, k, dtype=torch.int32, device=dev)
    for i in range(a.pool):
        step(i)
        logits_all[i].copy_(logits[0])
        routes[i].copy_(idx[0])
    torch.cuda.synchronize()

    ms_step, spread = time_steps(step, steps, warmup)

    # the expert phase as the forward runs it: the selecting gate/up GEMV, then
    # the down GEMV, each timed over back-to-back launches on its stream
    hbuf = torch.empty(k, I, dtype=torch.float32, device=dev)
    ybuf = torch.empty(k, H, dtype=torch.float32, device=dev)
    sel_i = torch.empty(1, k, dtype=torch.int32, device=dev)
    sel_w = torch.empty(1, k, dtype=torch.float32, device=dev)
    n = max(steps, 64)

    def gu_sel(i):
        j = (warmup + i) % a.pool
        moe.moe_mxfp4_gate_up_select(desc, pool[j:j + 1], logits_all[j:j + 1], k, codes, scales, sel_i, sel_w, hbuf)

    def down(i):
        j = (warmup + i) % a.pool
        moe.moe_mxfp4_down(desc, hbuf, routes[j], codes, scales, ybuf)

    def gu_given(i):
        j = (warmup + i) % a.pool
        moe.moe_mxfp4_gate_up(desc, pool[j:j + 1], routes[j], k, codes, scales, hbuf)

    gu_us = kernel_us(gu_sel, n, warmup)
    dn_us = kernel_us(down, n, warmup)
    gv_us = kernel_us(gu_given, n, warmup)
    gu_w = k * 2 * (I * H // 2 + I * H // 32)      # gate + up rows of the k experts
    dn_w = k * (H * I // 2 + H * I // 32)          # down rows of the k experts
    expert_bytes = k * w.expert_bytes              # 280,756,224 B
    assert gu_w + dn_w == expert_bytes
    ach = expert_bytes / ((gu_us + dn_us) * 1e-6) / 1e9
    roofline = {
        "bound": "hbm", "kernel": "expert phase as the forward runs it: k_gateup_ks (selecting) + k_down_ks",
        "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
        "traffic": sum_traffic([("k_gateup_ks", "decode"), ("k_down_ks", "decode")]),
        "bytes_per_launch": expert_bytes, "avg_launch_us": gu_us + dn_us,
        "kernels": {
            "k_gateup_ks_select": {"avg_launch_us": gu_us, "weight_bytes": gu_w,
                                     "frac": gu_w / (gu_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                                     "traffic": measured_traffic("k_gateup_ks", "decode")},
            "k_down_ks": {"avg_launch_us": dn_us, "weight_bytes": dn_w,
                          "frac": dn_w / (dn_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                          "traffic": measured_traffic("k_down_ks", "decode")},
            "k_gateup_ks_routes_given": {"avg_launch_us": gv_us,
                                           "frac": gu_w / (gv_us * 1e-6) / 1e9 / HBM_PEAK_GBS}},
    }
    # the same layer with the lossless scale4 side-car (2.88% fewer expert
    # bytes): bit-identical output, same steps and kernel timing
    s4 = None
    enc = moe.encode_scale4_layer(desc, scales)
    if enc is not None:
        desc4, scale4 = enc
        out4 = torch.empty(1, H, dtype=torch.float32, device=dev)
        for t in (0, 1):
            step(t)
            moe.moe_mxfp4_forward(desc4, pool[t:t + 1], wr, None, codes, scale4, k, out4, ws)
            torch.cuda.synchronize()
            if not torch.equal(out4.view(torch.int32), out.view(torch.int32)):
                refuse("scale4 forward differs from the 8-bit forward")

        def step4(i):
            x = pool[i % a.pool:i % a.pool + 1]
            moe.moe_mxfp4_forward(desc4, x, wr, None, codes, scale4, k, out4, ws)

        ms4, spread4 = time_steps(step4, steps, warmup)
        gu4 = kernel_us(lambda i: moe.moe_mxfp4_gate_up_select(
            desc4, pool[(warmup + i) % a.pool:(warmup + i) % a.pool + 1],
            logits_all[(warmup + i) % a.pool:(warmup + i) % a.pool + 1], k, codes, scale4, sel_i, sel_w, hbuf),
            n, warmup)
        dn4 = kernel_us(lambda i: moe.moe_mxfp4_down(desc4, hbuf, routes[(warmup + i) % a.pool], codes, scale4, ybuf),
                        n, warmup)
        eb4 = k * (sum(moe.packed_bytes(desc4)) // E)
        s4 = {"tokens_per_s": 1.0 / (ms4 * 1e-3), "ms_per_step": ms4, "ms_per_step_spread": spread4,
              "expert_bytes_per_token": eb4, "bytes_saved_frac": 1.0 - eb4 / expert_bytes,
              "expert_phase_us": {"k_gateup_ks_select": gu4, "k_down_ks": dn4},
              "expert_phase_GBps": eb4 / ((gu4 + dn4) * 1e-6) / 1e9,
              "expert_phase_frac": eb4 / ((gu4 + dn4) * 1e-6) / 1e9 / HBM_PEAK_GBS,
              "expert_phase_speedup": (gu_us + dn_us) / (gu4 + dn4), "bit_identical_to_8bit": True}
        log("decode scale4: %.2f us/step, expert phase %.1f + %.1f us (%.3f fewer bytes)" % (
            ms4 * 1e3, gu4, dn4, 1.0 - eb4 / expert_bytes))
        del scale4
    layer_bytes = expert_bytes + E * H * 4 + H * 2 + H * 4
    cfg = {"workload": "decode: T=1, H=7168, I=1536, E=896, k=16, bf16 x, all experts resident, "
                       "256-token rotating pool", "scale4": s4,
           "global_batch": 1, "layer_bytes_per_token": layer_bytes,
           "layer_GBps": layer_bytes / (ms_step * 1e-3) / 1e9, "layer_frac_hbm":
               layer_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, "expert_bytes_per_token": expert_bytes}
    log("decode: %.2f us/step, expert phase %.1f + %.1f us (frac %.3f)" % (ms_step * 1e3, gu_us, dn_us,
                                                                          ach / HBM_PEAK_GBS))
    return base_fields("MoE-layer tokens/s + achieved HBM GB/s (decode) / MFMA util (prefill)",
                       1.0 / (ms_step * 1e-3), "tokens/s", steps, warmup, ms_step, spread, cfg, roofline,
                       parity_obj([0, 1], *gate))


# --------------------------------------------------------------------------- matrix-core ceiling

def mfma_ceiling(reps=3, n_wg=1024, iters=2000):
    """The rate the matrix cores sustain on random operands with no memory
    traffic (moe_mfma_rate), per MFMA kind: TFLOP/s, best of reps launches of
    n_wg workgroups x 8 waves x iters x 8 MFMAs.  The ceiling under the clock
    the chip holds at that load, beside the nominal dense peaks."""
    import numpy as np
    import torch
    import mxfp4_routed_expert_fp32_amd as moe

    ops = torch.from_numpy(np.random.default_rng(2024).integers(0, 256, 65536, dtype=np.uint8)).to("cuda")
    sink = torch.empty(n_wg * 512, dtype=torch.float32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = {}
    for kind, (name, flops_per_mfma) in moe.MFMA_RATE_KINDS.items():
        moe.moe_mfma_rate(kind, ops, n_wg, 20, sink)
        best = None
        for _ in range(reps):
            torch.cuda.synchronize()
            e0.record()
            moe.moe_mfma_rate(kind, ops, n_wg, iters, sink)
            e1.record()
            torch.cuda.synchronize()
            sec = e0.elapsed_time(e1) * 1e-3
            best = sec if best is None else min(best, sec)
        out[name] = n_wg * 8 * iters * 8 * flops_per_mfma / best / 1e12
    return out


# --------------------------------------------------------------------------- batched decode / prefill

def bench_batch(a, ctx, name, steps, warmup):
    import numpy as np
    import torch

    import synth
    import synth.device as sd
    import mxfp4_routed_expert_fp32_amd as moe

    w = synth.WORKLOADS[name]
    desc = sd.desc_for(w)
    dev = "cuda"
    T, k, H, I, E = w.T, w.k, w.H, w.I, w.E
    codes, scales, wr = ctx.codes, ctx.scales, ctx.wr
    bias = sd.router_bias(w)
    nbatch = 8 if T <= 64 else 2                 # rotating batches of distinct tokens
    xs = [sd.tokens(w, range(b * T, (b + 1) * T)) for b in range(nbatch)]
    out = torch.empty(T, H, dtype=torch.float32, device=dev)
    logits = torch.empty(T, E, dtype=torch.float32, device=dev)
    idx = torch.empty(T, k, dtype=torch.int32, device=dev)
    wt = torch.empty(T, k, dtype=torch.float32, device=dev)
    ws = torch.empty(moe.workspace_bytes(desc, T, k), dtype=torch.uint8, device=dev)

    def step(i):
        moe.moe_mxfp4_forward(desc, xs[i % nbatch], wr, bias, codes, scales, k, out, ws, logits, idx, wt)

    # parity gate on sample tokens of batch 0: for the Zipf batch the tokens
    # also cover the hottest experts (every token selects the top three)
    step(0)
    torch.cuda.synchronize()
    idx_h = idx.cpu().numpy()
    if T <= 64:
        sample = sorted({0, 1, 17, 31, 40, 63} & set(range(T)))
    else:   # first and last pair of two expert blocks (sorted order), plus both ends
        flat = idx_h.reshape(-1)
        order = np.argsort(flat, kind="stable")
        offs = np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))])
        sample = {0, T - 1}
        for e in (int(np.argmax(np.diff(offs))), int(np.argmin(np.diff(offs)))):
            sample.update({int(order[offs[e]]) // k, int(order[offs[e + 1] - 1]) // k})
        sample = sorted(sample)
    b_h = None if bias is None else bias.cpu().numpy()
    gate = gate_tokens(w, synth.tokens_f32(w, sample), logits.cpu().numpy()[sample], idx_h[sample],
                       wt.cpu().numpy()[sample], out.cpu().numpy()[sample], wr.cpu().numpy(), bias=b_h)
    log("%s: parity ok on %d tokens (normwise %.3g, elementwise %.3g)" % (name, len(sample), *gate))

    unions, maxload = [], []
    for b in range(nbatch):
        step(b)
        torch.cuda.synchronize()
        ids = idx.cpu().numpy()
        unions.append(len(np.unique(ids)))
        maxload.append(int(np.bincount(ids.reshape(-1), minlength=E).max()))
    ms_step, spread = time_steps(step, steps, warmup)
    union = float(np.mean(unions))
    touched = union * w.expert_bytes + E * H * 4 + T * H * 2 + T * H * 4
    flops = 2.0 * T * k * 3 * H * I + 2.0 * T * E * H

    # the expert phase as the forward runs it (grouped gate/up, grouped down),
    # each kernel timed over back-to-back launches, over the sorted routes of
    # every rotating batch
    P_ = T * k
    mb = moe.max_expert_blocks(E, P_)
    nsw = moe.sort_workspace_bytes(E, T, k)
    sort_ws = torch.empty(nsw, dtype=torch.uint8, device=dev) if nsw else None
    stage = []
    for b in range(nbatch):
        step(b)
        offs = torch.empty(E + 1, dtype=torch.int32, device=dev)
        pairs = torch.empty(P_, dtype=torch.int32, device=dev)
        moe.moe_sort_by_expert(idx, E, offs, pairs, sort_ws)
        blocks = torch.empty(mb, 4, dtype=torch.int32, device=dev)
        nb = torch.empty(1, dtype=torch.int32, device=dev)
        moe.moe_expert_blocks(offs, P_, blocks, nb)
        stage.append((pairs, blocks, nb))
    hterm = torch.empty(2, P_, I, dtype=torch.bfloat16, device=dev)
    y = torch.empty(P_, H, dtype=torch.float32, device=dev)

    def gate_up(i):
        j = i % nbatch
        moe.moe_mxfp4_grouped_gate_up(desc, xs[j], k, stage[j][0], stage[j][1], stage[j][2], codes, scales, hterm)

    def down(i):
        j = i % nbatch
        moe.moe_mxfp4_grouped_down(desc, hterm, stage[j][0], stage[j][1], stage[j][2], codes, scales, y)

    nl = max(steps, 2 * nbatch)
    gu_us = kernel_us(gate_up, nl, warmup)
    dn_us = kernel_us(down, nl, warmup)
    del hterm, y
    exp_us = gu_us + dn_us
    wbytes = union * w.expert_bytes
    roof_common = {"avg_launch_us": exp_us,
                   "kernels": {"k_gateup_mfma": {"avg_launch_us": gu_us,
                                                 "traffic": measured_traffic("k_gateup_mfma", name)},
                               "k_down_mfma": {"avg_launch_us": dn_us,
                                               "traffic": measured_traffic("k_down_mfma", name)}},
                   "traffic": sum_traffic([("k_gateup_mfma", name), ("k_down_mfma", name)])}
    if name == "prefill4096":
        eflops = 2.0 * P_ * 3 * H * I
        ach = eflops / (exp_us * 1e-6) / 1e12
        roofline = {"bound": "mfma", "kernel": "expert phase as the forward runs it: k_gateup_mfma + k_down_mfma "
                                               "(bf16 MFMA, fp32 accumulate)",
                    "achieved": ach, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": ach / BF16_PEAK_TFLOPS,
                    "flops_per_launch": eflops, "frac_mxfp4_mfma_peak": ach / MXFP4_PEAK_TFLOPS,
                    "weight_bytes_per_launch": wbytes,
                    "frac_hbm_weights": wbytes / (exp_us * 1e-6) / 1e9 / HBM_PEAK_GBS, **roof_common}
        for kn, us, fl in (("k_gateup_mfma", gu_us, 4.0 * H * I * P_), ("k_down_mfma", dn_us, 2.0 * H * I * P_)):
            roofline["kernels"][kn]["frac"] = fl / (us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS
        ceil = mfma_ceiling()
        roofline["mfma_ceiling_measured_TFLOPs"] = ceil
        roofline["frac_of_measured_bf16_ceiling"] = ach / ceil["bf16"]
        log("%s: matrix cores on random operands: %s TFLOP/s" % (
            name, ", ".join("%s %.0f" % kv for kv in ceil.items())))
    else:
        ach = wbytes / (exp_us * 1e-6) / 1e9
        roofline = {"bound": "hbm", "kernel": "expert phase as the forward runs it: k_gateup_mfma + k_down_mfma",
                    "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                    "bytes_per_launch": wbytes, **roof_common}
        for kn, us, frac in (("k_gateup_mfma", gu_us, 2 / 3), ("k_down_mfma", dn_us, 1 / 3)):
            roofline["kernels"][kn]["frac"] = frac * wbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS
    tflops = flops / (ms_step * 1e-3) / 1e12
    cfg = {"workload": "%s: T=%d, H=%d, I=%d, E=%d, k=%d, bf16 x%s" % (
               name, T, H, I, E, k, ", Zipf(1.1) router bias" if bias is not None else ", uniform routing"),
           "global_batch": T, "experts_touched_mean": union, "max_expert_load": max(maxload),
           "touched_bytes_per_step": touched, "layer_GBps": touched / (ms_step * 1e-3) / 1e9,
           "algorithmic_TFLOPs": tflops, "frac_bf16_mfma_peak": tflops / BF16_PEAK_TFLOPS,
           "frac_mxfp4_mfma_peak": tflops / MXFP4_PEAK_TFLOPS}
    log("%s: %.3f ms/step, expert phase %.1f + %.1f us (frac %.3f)" % (name, ms_step, gu_us, dn_us,
                                                                       roofline["frac"]))
    res = base_fields("MoE-layer tokens/s (%s)" % name, T / (ms_step * 1e-3), "tokens/s", steps, warmup, ms_step,
                      spread, cfg, roofline, parity_obj(sample, *gate))
    del ws, out, logits
    torch.cuda.empty_cache()
    return res


# --------------------------------------------------------------------------- stack

def bench_stack(a, ctx, steps, warmup):
    import numpy as np
    import torch

    import synth
    import synth.device as sd
    import mxfp4_routed_expert_fp32_amd as moe
    from tests._stack_check import stack_layer_by_layer

    w = synth.WORKLOADS["stack12"]
    desc = sd.desc_for(w)
    dev = "cuda"
    t0 = time.time()
    layers = [(ctx.codes, ctx.scales, ctx.wr)]     # layer 0 is the decode layer (same seed)
    for l in range(1, w.layers):
        c, s = sd.upload_layer(w, l)
        layers.append((c, s, sd.router_w(w, l)))
    gam = [sd.gamma(w, l) for l in range(w.layers)]
    log("stack12: %d layers resident in %.1f s" % (w.layers, time.time() - t0))
    pool = sd.tokens(w, range(a.pool))
    # refusal gate: every layer against the oracle, from the GPU's residual before it
    (nw, ew), eager0, inputs = stack_layer_by_layer(w, desc, layers, gam, pool[0:1].contiguous(), 1, w.eps, w.k)
    log("stack12: parity ok, 12 layers (normwise %.3g, elementwise %.3g)" % (nw, ew))
    # next-layer route hint (prefetch only): the top-k of layer l's norm +
    # router on the input of layer l-1, against layer l's actual route (the
    # same function on layer l's input); overlap of the two sets
    hws = torch.empty(moe.route_hint_workspace_bytes(desc, 1, w.k), dtype=torch.uint8, device=dev)
    hint = torch.empty(1, w.k, dtype=torch.int32, device=dev)
    route = torch.empty(1, w.k, dtype=torch.int32, device=dev)
    overlaps = []
    for l in range(1, w.layers):
        moe.moe_route_hint(desc, torch.from_numpy(inputs[l - 1]).to(dev), gam[l], w.eps, layers[l][2], None, w.k,
                           hint, hws)
        moe.moe_route_hint(desc, torch.from_numpy(inputs[l]).to(dev), gam[l], w.eps, layers[l][2], None, w.k,
                           route, hws)
        torch.cuda.synchronize()
        overlaps.append(len(set(hint.cpu().numpy()[0].tolist()) & set(route.cpu().numpy()[0].tolist())) / w.k)
    log("stack12: next-layer hint overlap %.3f" % float(np.mean(overlaps)))
    x = torch.empty(1, w.H, dtype=torch.bfloat16, device=dev)
    resid = torch.empty(1, w.H, dtype=torch.float32, device=dev)
    ws = torch.empty(moe.stack_workspace_bytes(desc, 1, w.k), dtype=torch.uint8, device=dev)
    args = ([l[0] for l in layers], [l[1] for l in layers], [l[2] for l in layers], None, gam, w.eps)
    graph = moe.StackGraph(desc, *args, x, w.k, resid, ws)

    def step(i):
        x.copy_(pool[i % a.pool:i % a.pool + 1])
        graph.launch()

    def eager(i):
        x.copy_(pool[i % a.pool:i % a.pool + 1])
        moe.moe_mxfp4_stack_forward(desc, *args, x, w.k, resid, ws)

    step(0)
    torch.cuda.synchronize()
    if not np.array_equal(resid.cpu().numpy().view(np.uint32), eager0.view(np.uint32)):
        refuse("stack graph replay differs from the checked eager stack")
    ms_graph, spread = time_steps(step, steps, warmup)
    ms_eager, _ = time_steps(eager, max(10, steps // 4), 3)
    per_tok = w.layers * (w.k * w.expert_bytes + w.E * w.H * 4)
    gbps = per_tok / (ms_graph * 1e-3) / 1e9
    cfg = {"workload": "stack12: 12 layers x (RMSNorm eps=1e-6 + MoE H=7168 I=1536 E=896 k=16 + residual), T=1, "
                       "hipGraph replay, 256-token rotating pool",
           "global_batch": 1, "bytes_per_token": per_tok, "GBps": gbps, "ms_per_token_eager": ms_eager,
           "graph_equals_eager": True,
           "route_hint": {"mean_overlap": float(np.mean(overlaps)), "min_overlap": float(np.min(overlaps)),
                          "layers": w.layers - 1, "tokens": 1,
                          "what": "fraction of layer l's routed experts that the hint computed from layer l-1's "
                                  "input predicts (prefetch only; never used for compute)"}}
    roofline = {"bound": "hbm", "kernel": "whole step (12 layers, graph replay)", "achieved": gbps,
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbps / HBM_PEAK_GBS, "traffic": None,
                "bytes_per_launch": per_tok, "avg_launch_us": ms_graph * 1e3}
    graph.close()
    log("stack12: %.3f ms/token (eager %.3f), frac %.3f" % (ms_graph, ms_eager, gbps / HBM_PEAK_GBS))
    return base_fields("12-layer MoE stack decode tokens/s", 1.0 / (ms_graph * 1e-3), "tokens/s", steps, warmup,
                       ms_graph, spread, cfg, roofline, parity_obj([0], nw, ew))


# --------------------------------------------------------------------------- host-streamed decode

HOST_LINK_PEAK_GBS = 64.0   # PCIe 5.0 x16, one direction


def bench_streamed(a, ctx, steps):
    """Single-token decode of the model-shape layer with its experts in host
    memory and a 256-slot device residency cache: each step routes on the
    device, reads the route back, plans, uploads the misses and runs the
    experts on the cache's slots.  Measured with pageable host memory (two
    pinned staging slabs) and with pinned host memory (direct DMA)."""
    import numpy as np
    import torch

    import synth
    import synth.device as sd
    import mxfp4_routed_expert_fp32_amd as moe

    w = synth.WORKLOADS["decode"]
    desc = sd.desc_for(w)
    dev = "cuda"
    k, H, E = w.k, w.H, w.E
    t0 = time.time()
    host_c, host_s = synth.experts(w, 0)          # 15.72 GB of pageable host memory
    log("decode_streamed: layer 0 in host memory in %.1f s" % (time.time() - t0))
    pool = sd.tokens(w, range(a.pool))
    out = torch.empty(1, H, dtype=torch.float32, device=dev)
    ref = torch.empty(1, H, dtype=torch.float32, device=dev)
    ws_r = torch.empty(moe.workspace_bytes(desc, 1, k), dtype=torch.uint8, device=dev)
    res = {}
    for mode in ("pageable", "pinned"):
        if mode == "pinned":
            t0 = time.time()
            pc = torch.empty(host_c.size, dtype=torch.uint8, pin_memory=True)
            ps = torch.empty(host_s.size, dtype=torch.uint8, pin_memory=True)
            pc.numpy()[:] = host_c
            ps.numpy()[:] = host_s
            src = (pc, ps)
            log("decode_streamed: pinned copy in %.1f s" % (time.time() - t0))
        else:
            src = (host_c, host_s)
        cache = moe.ExpertCache(desc, 1, capacity=256)
        ws = torch.empty(cache.workspace_bytes(1, k), dtype=torch.uint8, device=dev)
        # gate: bit-identical to the all-resident forward on two tokens
        for t in (0, 1):
            x = pool[t:t + 1]
            moe.moe_mxfp4_forward(desc, x, ctx.wr, None, ctx.codes, ctx.scales, k, ref, ws_r)
            cache.layer_forward(0, x, ctx.wr, None, src[0], src[1], k, out, ws, pinned=(mode == "pinned"))
            torch.cuda.synchronize()
            if not torch.equal(out.view(torch.int32), ref.view(torch.int32)):
                refuse("streamed layer differs from the resident forward")
        s0 = cache.stats()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            x = pool[(2 + i) % a.pool:(2 + i) % a.pool + 1]
            cache.layer_forward(0, x, ctx.wr, None, src[0], src[1], k, out, ws, pinned=(mode == "pinned"))
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        s1 = cache.stats()
        up = s1["bytes_uploaded"] - s0["bytes_uploaded"]
        hits, misses = s1["hits"] - s0["hits"], s1["misses"] - s0["misses"]
        gbps = up / dt / 1e9
        res[mode] = {"tokens_per_s": steps / dt, "ms_per_token": dt * 1e3 / steps, "host_link_GBps": gbps,
                     "frac_host_link": gbps / HOST_LINK_PEAK_GBS, "hits": hits, "misses": misses,
                     "bytes_uploaded": up, "capacity_slots": cache.capacity}
        log("decode_streamed %s: %.2f ms/token, %.1f GB/s host link, %d hits / %d misses" % (
            mode, dt * 1e3 / steps, gbps, hits, misses))
        cache.close()
        del src
    best = res["pinned"]
    cfg = {"workload": "decode_streamed: decode workload (T=1, K3 shape) with the 896 experts in host memory and a "
                       "256-slot device residency cache (LRU), 256-token rotating pool",
           "global_batch": 1, "pageable": res["pageable"], "pinned": res["pinned"]}
    roofline = {"bound": "host-link", "kernel": "expert uploads host -> device (pinned host memory, direct DMA)",
                "achieved": best["host_link_GBps"], "peak": HOST_LINK_PEAK_GBS, "unit": "GB/s",
                "frac": best["host_link_GBps"] / HOST_LINK_PEAK_GBS, "traffic": None,
                "bytes_per_launch": best["bytes_uploaded"] / steps, "avg_launch_us": best["ms_per_token"] * 1e3}
    return base_fields("MoE-layer tokens/s (decode, experts streamed from host memory)", best["tokens_per_s"],
                       "tokens/s", steps, 0, best["ms_per_token"], None, cfg, roofline,
                       {"tokens_checked": [0, 1], "bit_identical_to_resident_forward": True})


# --------------------------------------------------------------------------- packed-int8 spine GEMV

def bench_int8(a, steps, warmup):
    """The resident-spine GEMV of packed-int8 rows with fp16 row scales at the
    pages' 12288 x 7168 shape, one fp32 token; launches rotate over four
    distinct matrices (352 MB, more than the 256 MB last-level cache)."""
    import numpy as np
    import torch

    import oracle
    import synth
    import mxfp4_routed_expert_fp32_amd as moe
    from tests import _parity as P

    N, K, NM = 12288, 7168, 4
    dev = "cuda"
    mats = []
    for m in range(NM):
        q, s = synth.int8_rows(100 + m, N, K)
        mats.append((q, s, torch.from_numpy(q).to(dev), torch.from_numpy(s.view(np.int16)).to(dev)))
    x = synth.normal_f32(synth.key(5, 0, 1, 777), K).reshape(1, K)
    xd = torch.from_numpy(x).to(dev)
    y = torch.empty(1, N, dtype=torch.float32, device=dev)
    # gate: every row of matrix 0 against the oracle, both readings
    moe.moe_int8_gemv(mats[0][2], mats[0][3], xd, y)
    torch.cuda.synchronize()
    ref = oracle.int8_gemv(mats[0][0], mats[0][1], x)
    W = oracle.int8_dequant(mats[0][0], mats[0][1]).astype(np.float64)
    A = np.abs(x).astype(np.float64) @ np.abs(W).T
    got = y.cpu().numpy()
    nw_, ew_ = float(P.normwise_err(got, ref).max()), P.elementwise_ratio(got, ref, A)
    if not (nw_ <= P.OUT_TOL and ew_ <= P.OUT_TOL):
        refuse("int8 GEMV: normwise %g, elementwise %g" % (nw_, ew_))
    log("spine_int8: parity ok (normwise %.3g, elementwise %.3g)" % (nw_, ew_))
    bytes_per = N * K + N * 2 + K * 4 + N * 4
    sweep = {}
    for rpw in (0, 16, 24, 32, 40, 56, 64):
        us = kernel_us(lambda i: moe.moe_int8_gemv(mats[i % NM][2], mats[i % NM][3], xd, y, rows_per_workgroup=rpw),
                       max(steps, 4 * NM), warmup)
        sweep[rpw] = us
    best = min(sweep, key=sweep.get)
    us = sweep[0]
    ach = bytes_per / (us * 1e-6) / 1e9
    out = torch.empty(N, K, dtype=torch.float32, device=dev)
    dq_us = kernel_us(lambda i: moe.moe_int8_dequant(mats[i % NM][2], mats[i % NM][3], out), max(steps, 4 * NM),
                      warmup)
    dq_bytes = N * K + N * 2 + N * K * 4
    log("spine_int8: %.1f us per GEMV (%.0f GB/s, frac %.3f); dequant export %.1f us (%.0f GB/s)" % (
        us, ach, ach / HBM_PEAK_GBS, dq_us, dq_bytes / (dq_us * 1e-6) / 1e9))
    cfg = {"workload": "spine_int8: packed-int8 rows with fp16 row scales, 12288 x 7168, one fp32 token, four "
                       "rotating matrices", "global_batch": 1,
           "rows_per_workgroup_sweep_us": {str(k_): v for k_, v in sweep.items()}, "best_rows_per_workgroup": best,
           "dequant_export": {"avg_launch_us": dq_us, "bytes_per_launch": dq_bytes,
                              "GBps": dq_bytes / (dq_us * 1e-6) / 1e9,
                              "frac": dq_bytes / (dq_us * 1e-6) / 1e9 / HBM_PEAK_GBS}}
    roofline = {"bound": "hbm", "kernel": "k_int8_gemv (default split)", "achieved": ach, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": ach / HBM_PEAK_GBS, "traffic": measured_traffic("k_int8_gemv", "spine_int8"),
                "bytes_per_launch": bytes_per,
                "avg_launch_us": us}
    return base_fields("packed-int8 spine GEMV rows/s (12288 x 7168)", N / (us * 1e-6), "rows/s", max(steps, 4 * NM),
                       warmup, us * 1e-3, None, cfg, roofline, parity_obj([0], nw_, ew_))


# --------------------------------------------------------------------------- CPU baseline

def cpu_info():
    model, mhz = None, []
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name") and model is None:
                model = line.split(":", 1)[1].strip()
            elif line.startswith("cpu MHz"):
                mhz.append(float(line.split(":", 1)[1]))
    except OSError:
        pass
    return model, (statistics.mean(mhz) if mhz else None)


def cpu_baseline(w, seconds):
    """The oracle as it is, on the host cores, on whole tokens of the decode
    workload until `seconds` of oracle time have been spent (at least 3
    tokens, one oracle call each); per-call times give the median and range."""
    import numpy as np

    import oracle
    import synth

    wr = synth.router_w(w)
    bias = synth.router_bias(w)
    cores = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        cores = min(cores, int(os.environ["OMP_NUM_THREADS"]))
    model, mhz = cpu_info()
    times = []
    while len(times) < 3 or sum(times) < seconds:
        t = 100000 + len(times)
        x = synth.tokens_f32(w, [t])
        sel = np.unique(oracle.topk(oracle.router_logits(x, wr, bias), w.k))
        ex = {int(e): synth.expert(w, int(e)) for e in sel}
        t0 = time.perf_counter()
        oracle.moe_forward(x, wr, ex, w.H, w.I, w.k, bias=bias, nthreads=cores)
        times.append(time.perf_counter() - t0)
        if len(times) >= 512:
            break
    spent = sum(times)
    return {"value": len(times) / spent, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "median_tokens_per_s": 1.0 / statistics.median(times), "min_tokens_per_s": 1.0 / max(times),
            "max_tokens_per_s": 1.0 / min(times), "cpu_model": model, "cpu_mhz_mean": mhz,
            "sample": "%d tokens of the decode workload, one oracle call each (router, top-k, 16 experts "
                      "dequantised and applied, combine), %.1f s of oracle time; expert generation not timed"
                      % (len(times), spent)}


# --------------------------------------------------------------------------- main

def main():
    a = parse()
    if a.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % a.gpus, file=sys.stderr)
        sys.exit(2)
    names = WORKLOADS if a.workload == "all" else [a.workload]
    primary = names[0]
    ctx = Ctx()
    results = {}
    for name in names:
        steps, warmup = DEFAULT_STEPS[name]
        if name == primary:
            steps = steps if a.steps is None else a.steps
            warmup = warmup if a.warmup is None else a.warmup
        if name == "decode":
            results[name] = bench_decode(a, ctx, steps, warmup)
        elif name == "stack12":
            results[name] = bench_stack(a, ctx, steps, warmup)
        elif name == "decode_streamed":
            results[name] = bench_streamed(a, ctx, steps)
        elif name == "spine_int8":
            results[name] = bench_int8(a, steps, warmup)
        else:
            results[name] = bench_batch(a, ctx, name, steps, warmup)
    res = results[primary]
    if len(names) > 1:
        res["workloads"] = {n: results[n] for n in names[1:]}
    res["cpu_baseline"] = None
    if not a.no_cpu_baseline:
        import synth
        res["cpu_baseline"] = cpu_baseline(synth.WORKLOADS["decode"], a.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
