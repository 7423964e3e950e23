"""The router trace writer and reader (host code, no GPU): records round-trip
(ids and the exact fp32 weight bits), both write modes, the size cap, symlink
refusal, and strict parsing for offline warming counts."""
import json
import os

import numpy as np
import pytest

import mxfp4_routed_expert_fp32_amd as moe

pytestmark = pytest.mark.skipif(not os.path.exists(moe.LIB_PATH), reason="libmoe_mxfp4.so not built")


def routes(rng, T, E, k):
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.dirichlet(np.ones(k), T).astype(np.float32)
    w[0, 0] = np.float32(-0.0)                        # a sign bit that a decimal round trip could lose
    w[0, 1] = np.float32(1e-45)                       # a subnormal
    return ids, w


@pytest.mark.parametrize("mode", [moe.MOE_TRACE_BUFFERED, moe.MOE_TRACE_SYNC])
def test_trace_round_trip_and_counts(tmp_path, mode):
    rng = np.random.default_rng(mode)
    L, E, k = 3, 40, 8
    path = str(tmp_path / "trace.jsonl")
    tr = moe.RouteTrace(path, mode)
    recs = []
    for step in range(5):
        for layer in range(L):
            ids, w = routes(rng, 4, E, k)
            tr.record(layer, 100 * step, ids, w)
            recs.append((layer, 100 * step, ids, w))
    tr.close()
    lines = open(path).read().splitlines()
    assert len(lines) == 5 * L * 4
    i = 0
    want_counts = np.zeros((L, E), np.int64)
    for layer, pos, ids, w in recs:
        for t in range(ids.shape[0]):
            d = json.loads(lines[i])
            i += 1
            assert d["layer"] == layer and d["pos"] == pos + t
            assert d["ids"] == ids[t].tolist()
            assert [int(h, 16) for h in d["w"]] == w[t].view(np.uint32).tolist()
            np.add.at(want_counts[layer], ids[t], 1)
    counts, n = moe.trace_count(path, L, E)
    assert n == len(lines) and np.array_equal(counts, want_counts)


def test_trace_refuses_symlink_and_non_regular(tmp_path):
    target = tmp_path / "real.jsonl"
    target.write_text("")
    link = tmp_path / "link.jsonl"
    os.symlink(target, link)
    for p in (link, tmp_path):                        # a symlink, a directory
        with pytest.raises(moe.MoeError) as e:
            moe.RouteTrace(str(p))
        assert e.value.status == -15
    with pytest.raises(moe.MoeError) as e:
        moe.trace_count(str(link), 1, 8)
    assert e.value.status == -15


def test_trace_size_cap(tmp_path):
    path = str(tmp_path / "capped.jsonl")
    rng = np.random.default_rng(7)
    ids, w = routes(rng, 1, 64, 16)
    tr = moe.RouteTrace(path, moe.MOE_TRACE_BUFFERED, max_bytes=1000)
    tr.record(0, 0, ids, w)                           # one line of about 300 bytes
    tr.record(0, 1, ids, w)
    tr.record(0, 2, ids, w)
    with pytest.raises(moe.MoeError) as e:            # the fourth would pass 1000 bytes
        tr.record(0, 3, ids, w)
    assert e.value.status == -15
    with pytest.raises(moe.MoeError):                 # the trace stays stopped
        tr.record(0, 4, ids, w)
    with pytest.raises(moe.MoeError):                 # and close reports the failure
        tr.close()
    assert os.path.getsize(path) <= 1000
    counts, n = moe.trace_count(path, 1, 64)
    assert n == 3 and counts.sum() == 3 * 16


@pytest.mark.parametrize("bad", [
    '{"layer":0,"pos":0,"ids":[1,2],"w":["3f800000"]}\n',            # fewer weights than ids
    '{"layer":0,"pos":0,"ids":[1,99],"w":["3f800000","00000000"]}\n',  # id out of range
    '{"layer":5,"pos":0,"ids":[1],"w":["3f800000"]}\n',              # layer out of range
    '{"layer":0,"pos":0,"ids":[1],"w":["3F800000"]}\n',              # not lowercase hex
    '{"layer":0,"pos":0,"ids":[1],"w":["3f800000"]}',                 # unterminated
    '{"layer":0,"pos":0,"ids":[1],"w":["3f800000"]} \n',             # trailing bytes
    '{"layer":0,"pos":0,"ids":[' + ",".join(["1"] * 1200) + '],"w":[]}\n',  # over-long line
])
def test_trace_count_rejects_malformed(tmp_path, bad):
    p = tmp_path / "bad.jsonl"
    p.write_text('{"layer":0,"pos":0,"ids":[3],"w":["3f800000"]}\n' + bad)
    with pytest.raises(moe.MoeError) as e:
        moe.trace_count(str(p), 2, 32)
    assert e.value.status == -15
