"""The expert residency cache (host-streamed experts, a device slot pool with
one LRU order across layers): plan order and accounting against a host model
of the policy, slot contents after uploads, the state rules, poisoning, and
layer calls whose output is bit-identical to the all-resident forward while
the cache holds fewer experts than the calls touch."""
import os

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


class LRUModel:
    """The cache's policy in plain Python: hits keep their slots; misses in
    route order take the lowest free slot, else the least recently used slot
    (lowest index on ties) that the plan does not use."""

    def __init__(self, cap):
        self.cap = cap
        self.owner = [None] * cap
        self.last = [0] * cap
        self.slot_of = {}
        self.tick = 0
        self.hits = self.misses = self.evictions = self.prefetched = 0

    def plan(self, layer, ids, prefetch=False):
        uni = list(dict.fromkeys(int(i) for i in ids))
        self.tick += 1
        inplan = set()
        for e in uni:
            s = self.slot_of.get((layer, e))
            if s is not None:
                inplan.add(s)
                self.last[s] = self.tick
                if not prefetch:
                    self.hits += 1
        misses = []
        for e in uni:
            if (layer, e) in self.slot_of:
                continue
            free = [s for s in range(self.cap) if s not in inplan and self.owner[s] is None]
            if free:
                s = free[0]
            else:
                s = min((s for s in range(self.cap) if s not in inplan), key=lambda q: (self.last[q], q))
                del self.slot_of[self.owner[s]]
                self.evictions += 1
            self.owner[s] = (layer, e)
            self.slot_of[(layer, e)] = s
            self.last[s] = self.tick
            inplan.add(s)
            misses.append(e)
            if prefetch:
                self.prefetched += 1
            else:
                self.misses += 1
        slots = [self.slot_of[(layer, int(i))] for i in ids]
        return slots, misses


def host_layers(w, n_layers):
    ce, se = w.code_bytes_per_expert, w.scale_bytes_per_expert
    out = []
    for l in range(n_layers):
        c, s = synth.experts(w, l)
        out.append((c, s, [c[e * ce:(e + 1) * ce] for e in range(w.E)], [s[e * se:(e + 1) * se] for e in range(w.E)]))
    return out


def assert_slot_holds(cache, slot, codes_e, scales_e, w):
    """The slot's gate and down matrices dequantise to the source expert's."""
    mc, ms = w.I * w.H // 2, w.I * w.H // 32
    for m, (rows, cols) in ((0, (w.I, w.H)), (2, (w.H, w.I))):
        out = torch.empty(rows, cols, dtype=torch.float32, device=DEV)
        moe.lib().moe_mxfp4_dequant(moe.ctypes.byref(cache.slot_desc), cache.slot_codes, cache.slot_scales, slot, m,
                                    moe.ctypes.c_void_p(out.data_ptr()), moe._stream(None))
        torch.cuda.synchronize()
        ref = oracle.dequant(codes_e[m * mc:(m + 1) * mc], scales_e[m * ms:(m + 1) * ms], rows, cols)
        assert np.array_equal(P.bits(out.cpu().numpy()), P.bits(ref)), (slot, m)


def test_cache_plan_order_lru_and_state_rules():
    w = synth.Workload("rc", 75, 1, 512, 256, 16, 2, "bf16", weight_seed=8600)
    desc = sd.desc_for(w)
    layers = host_layers(w, 2)
    cache = moe.ExpertCache(desc, 2, capacity=4)
    assert cache.capacity == 4
    model = LRUModel(4)
    seq = [(0, [3, 5, 3], False), (0, [5, 7], False), (1, [3, 9], False), (1, [9, 11], False),
           (0, [5, 2], False), (1, [12, 13], True), (0, [7, 5], False), (1, [13, 3], False)]
    for layer, ids, pre in seq:
        slots, miss = cache.plan(layer, np.array(ids, np.int32), prefetch=pre)
        m_slots, m_miss = model.plan(layer, ids, prefetch=pre)
        assert list(miss) == m_miss, (layer, ids)
        if not pre:
            assert list(slots) == m_slots, (layer, ids)
        cache.finish([layers[layer][2][e] for e in miss], [layers[layer][3][e] for e in miss])
        torch.cuda.synchronize()
        for e in dict.fromkeys(ids):
            assert_slot_holds(cache, model.slot_of[(layer, e)], layers[layer][2][e], layers[layer][3][e], w)
    st = cache.stats()
    assert (st["hits"], st["misses"], st["evictions"], st["prefetched"]) == (
        model.hits, model.misses, model.evictions, model.prefetched)
    assert st["bytes_uploaded"] == (model.misses + model.prefetched) * w.expert_bytes
    assert st["plans"] == len(seq) and st["poisoned"] == 0
    # state rules: one frozen plan at a time; finish needs a plan; cancel frees the misses' slots
    cache.plan(0, np.array([1], np.int32))
    with pytest.raises(moe.MoeError) as e:
        cache.plan(0, np.array([4], np.int32))
    assert e.value.status == -14
    cache.cancel()
    with pytest.raises(moe.MoeError) as e:
        cache.finish([], [])
    assert e.value.status == -14
    with pytest.raises(moe.MoeError) as e:                       # union above the capacity
        cache.plan(0, np.arange(5, dtype=np.int32))
    assert e.value.status == -7
    with pytest.raises(moe.MoeError) as e:                       # id outside [0, E)
        cache.plan(0, np.array([16], np.int32))
    assert e.value.status == -11
    with pytest.raises(moe.MoeError) as e:                       # layer outside [0, n_layers)
        cache.plan(2, np.array([1], np.int32))
    assert e.value.status == -11
    cache.close()


def test_cache_poisoned_after_failed_upload():
    """A failed upload (forced from the host: the hook makes upload 2 report a
    failure) poisons the cache; every later call is refused."""
    w = synth.Workload("rp", 76, 1, 256, 256, 8, 2, "bf16", weight_seed=8700)
    desc = sd.desc_for(w)
    layers = host_layers(w, 1)
    os.environ["MOE_CACHE_FAIL_UPLOAD"] = "2"
    try:
        cache = moe.ExpertCache(desc, 1, capacity=4)
    finally:
        del os.environ["MOE_CACHE_FAIL_UPLOAD"]
    _, miss = cache.plan(0, np.array([0, 1], np.int32))
    cache.finish([layers[0][2][e] for e in miss], [layers[0][3][e] for e in miss])
    _, miss = cache.plan(0, np.array([2, 3], np.int32))
    with pytest.raises(moe.MoeError) as e:
        cache.finish([layers[0][2][e] for e in miss], [layers[0][3][e] for e in miss])
    assert e.value.status == -13
    for call in (lambda: cache.plan(0, np.array([0], np.int32)), lambda: cache.finish([], [])):
        with pytest.raises(moe.MoeError) as e:
            call()
        assert e.value.status == -13
    assert cache.stats()["poisoned"] == 1
    torch.cuda.synchronize()
    cache.close()


@pytest.mark.parametrize("pinned", [False, True])
def test_cache_layer_forward_equals_resident_forward(pinned):
    """Two layers streamed through a 12-slot cache (each call's union fits,
    the calls together touch far more experts): decode with one bf16 token, the prefill form with several bf16
    tokens, and the fp32 decode form, each bit-identical to the all-resident
    forward; hits and misses follow the host model exactly."""
    H, I, E, k, L = 512, 256, 24, 4, 2
    w = synth.Workload("rf", 77, 6, H, I, E, k, "bf16", weight_seed=8800)
    wf = synth.Workload("rf", 77, 6, H, I, E, k, "f32", weight_seed=8800)
    desc = sd.desc_for(w)
    layers = host_layers(w, L)
    resident = [sd.upload_layer(w, l) for l in range(L)]
    wrs = [sd.router_w(w, l) for l in range(L)]
    if pinned:
        src = [(torch.from_numpy(c).pin_memory(), torch.from_numpy(s).pin_memory()) for c, s, _, _ in layers]
    else:
        src = [(c, s) for c, s, _, _ in layers]
    cache = moe.ExpertCache(desc, L, capacity=12)
    model = LRUModel(12)
    calls = [(0, [0], w), (1, [1], w), (0, [2, 3, 4], w), (1, [7, 8, 9], wf), (0, [0], w), (1, [1], w),
             (1, [10, 11, 12], w), (0, [16, 17], wf), (0, [0], w), (1, [5, 6], w), (0, [13, 14, 15], w)]
    for layer, toks, ww in calls:
        x = sd.tokens(ww, toks)
        T = len(toks)
        ref = torch.empty(T, H, dtype=torch.float32, device=DEV)
        ridx = torch.empty(T, k, dtype=torch.int32, device=DEV)
        rw = torch.empty(T, k, dtype=torch.float32, device=DEV)
        ws = torch.empty(moe.workspace_bytes(desc, T, k), dtype=torch.uint8, device=DEV)
        moe.moe_mxfp4_forward(desc, x, wrs[layer], None, resident[layer][0], resident[layer][1], k, ref, ws, None,
                              ridx, rw)
        out = torch.empty(T, H, dtype=torch.float32, device=DEV)
        cidx = torch.empty(T, k, dtype=torch.int32, device=DEV)
        cw = torch.empty(T, k, dtype=torch.float32, device=DEV)
        cws = torch.empty(cache.workspace_bytes(T, k), dtype=torch.uint8, device=DEV)
        cache.layer_forward(layer, x, wrs[layer], None, src[layer][0], src[layer][1], k, out, cws, cidx, cw,
                            pinned=pinned)
        torch.cuda.synchronize()
        assert np.array_equal(cidx.cpu().numpy(), ridx.cpu().numpy())
        assert np.array_equal(P.bits(cw.cpu().numpy()), P.bits(rw.cpu().numpy()))
        assert np.array_equal(P.bits(out.cpu().numpy()), P.bits(ref.cpu().numpy())), (layer, toks)
        model.plan(layer, ridx.cpu().numpy().reshape(-1))
    st = cache.stats()
    assert (st["hits"], st["misses"], st["evictions"]) == (model.hits, model.misses, model.evictions)
    assert st["misses"] > cache.capacity and st["hits"] > 0 and st["evictions"] > 0
    cache.close()


def streamed_stack(cache, desc, host, wrs, gam, eps, x, k, prefetch=False, trace=None, hint_log=None):
    """The pre-norm stack with every layer's experts streamed through the
    cache: r = x; per layer, n = RMSNorm(r), r += experts(n) on the cache's
    slots.  With prefetch, the next layer's hint (from this layer's input r)
    is prefetched into the cache after the layer's call is enqueued."""
    T, H = x.shape
    L = len(host)
    r = x.float().contiguous()
    n = torch.empty_like(r)
    out = torch.empty_like(r)
    idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    wt = torch.empty(T, k, dtype=torch.float32, device=DEV)
    ws = torch.empty(cache.workspace_bytes(T, k), dtype=torch.uint8, device=DEV)
    hws = torch.empty(moe.route_hint_workspace_bytes(desc, T, k), dtype=torch.uint8, device=DEV)
    hint = torch.empty(T, k, dtype=torch.int32, device=DEV)
    for l in range(L):
        if prefetch and l + 1 < L:
            moe.moe_route_hint(desc, r, gam[l + 1], eps, wrs[l + 1], None, k, hint, hws)
        moe.moe_rmsnorm(r, gam[l], eps, n)
        cache.layer_forward(l, n, wrs[l], None, host[l][0], host[l][1], k, out, ws, idx, wt)
        if trace is not None:
            torch.cuda.synchronize()
            trace.record(l, 0, idx.cpu().numpy(), wt.cpu().numpy())
        if prefetch and l + 1 < L:
            h = hint.cpu().numpy()
            _, miss = cache.plan(l + 1, h.reshape(-1), prefetch=True)
            cache.finish([host[l + 1][2][e] for e in miss], [host[l + 1][3][e] for e in miss])
            if hint_log is not None:
                hint_log.append((l + 1, h))
        moe.moe_residual_add(r, out)
    torch.cuda.synchronize()
    return r.cpu().numpy()


def test_route_hint_and_hint_prefetch_keep_outputs(tmp_path):
    """The next-layer hint is the exact top-k of the next layer's norm + router
    on the given activation (bit-equal to the stage entries); a three-layer
    stack streamed through a small cache gives the resident stack's bits with
    and without hint-driven prefetch, and prefetch turns demand misses into
    hits.  The trace of the routes read back counts every routed expert."""
    H, I, E, k, L, T = 512, 256, 32, 4, 3, 2
    w = synth.Workload("hp", 78, T, H, I, E, k, "bf16", weight_seed=8900)
    desc = sd.desc_for(w)
    layers = host_layers(w, L)
    host = [(c, s, cs, ss) for c, s, cs, ss in layers]
    wrs = [sd.router_w(w, l) for l in range(L)]
    gam = [sd.gamma(w, l) for l in range(L)]
    x = sd.tokens(w, range(T))
    # the hint against the stage entries on the same activation
    r = torch.from_numpy(np.random.default_rng(5).standard_normal((T, H)).astype(np.float32)).to(DEV)
    hint = torch.empty(T, k, dtype=torch.int32, device=DEV)
    hws = torch.empty(moe.route_hint_workspace_bytes(desc, T, k), dtype=torch.uint8, device=DEV)
    moe.moe_route_hint(desc, r, gam[1], w.eps, wrs[1], None, k, hint, hws)
    n = torch.empty_like(r)
    moe.moe_rmsnorm(r, gam[1], w.eps, n)
    lg = torch.empty(T, E, dtype=torch.float32, device=DEV)
    moe.moe_router_logits(desc, n, wrs[1], None, lg)
    idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    wt = torch.empty(T, k, dtype=torch.float32, device=DEV)
    moe.moe_topk_softmax(lg, k, idx, wt)
    torch.cuda.synchronize()
    assert np.array_equal(hint.cpu().numpy(), idx.cpu().numpy())
    # the resident stack
    resident = [sd.upload_layer(w, l) for l in range(L)]
    resid = torch.empty(T, H, dtype=torch.float32, device=DEV)
    sws = torch.empty(moe.stack_workspace_bytes(desc, T, k), dtype=torch.uint8, device=DEV)
    moe.moe_mxfp4_stack_forward(desc, [c for c, _ in resident], [s for _, s in resident], wrs, None, gam, w.eps, x, k,
                                resid, sws)
    torch.cuda.synchronize()
    want = resid.cpu().numpy()
    got, stats = {}, {}
    for pre in (False, True):
        cache = moe.ExpertCache(desc, L, capacity=8)
        tr = moe.RouteTrace(str(tmp_path / ("t%d.jsonl" % pre)))
        log = []
        got[pre] = streamed_stack(cache, desc, host, wrs, gam, w.eps, x, k, prefetch=pre, trace=tr, hint_log=log)
        tr.close()
        stats[pre] = cache.stats()
        cache.close()
        counts, nrec = moe.trace_count(str(tmp_path / ("t%d.jsonl" % pre)), L, E)
        assert nrec == L * T and counts.sum() == L * T * k
        assert np.array_equal(P.bits(got[pre]), P.bits(want)), "prefetch=%s" % pre
    assert stats[True]["prefetched"] > 0
    assert stats[True]["misses"] < stats[False]["misses"]
