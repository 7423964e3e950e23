"""The synthetic input generator: determinism, distributions, independence of items."""
import json
import os

import numpy as np

import synth
from tests.golden import make_synth_hashes


def test_golden_hashes(golden_dir):
    with open(os.path.join(golden_dir, "synth_sha256.json")) as f:
        ref = json.load(f)
    assert make_synth_hashes.digests() == ref


def test_expert_regenerates_alone():
    w = synth.WORKLOADS["tiny"]
    c, s = synth.experts(w)
    for e in (0, 5, 7):
        ce, se = synth.expert(w, e)
        assert np.array_equal(ce, c[e * w.code_bytes_per_expert:(e + 1) * w.code_bytes_per_expert])
        assert np.array_equal(se, s[e * w.scale_bytes_per_expert:(e + 1) * w.scale_bytes_per_expert])


def test_distributions():
    w = synth.WORKLOADS["tiny"]
    c, s = synth.experts(w)
    nib = np.concatenate([c & 0xF, c >> 4])
    counts = np.bincount(nib, minlength=16)
    assert counts.min() > 0.9 * nib.size / 16
    assert set(np.unique(s)) == {119, 120, 121, 122, 123}
    x = synth.normal_f32(synth.key(1, 0, 1, 0), 200000)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    wr = synth.router_w(synth.WORKLOADS["tiny"])
    assert abs(wr.std() - 1 / 16) < 0.003
    g = synth.gamma(synth.WORKLOADS["stack12"], 0)
    assert g.min() >= 0.5 and g.max() < 1.5


def test_bf16_rounding_is_rne():
    a = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5], np.float32)
    b = synth.f32_to_bf16_bits(a)
    assert list(b) == [0x3F80, 0x3F80, 0x3F82, 0x3F80, 0xC020]


def test_zipf_bias_skews_selection():
    w = synth.WORKLOADS["decode64_zipf"]
    b = synth.router_bias(w)
    rank = synth.zipf_rank(w)
    assert b[rank == 1][0] > 5 and b[rank == w.E][0] < -2.5
    assert np.all(np.diff(b[np.argsort(rank)]) <= 0)
