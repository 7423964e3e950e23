"""Writes synth_sha256.json: SHA-256 of generated input tensors, so that a change
to the synthetic input generator is noticed.  Calls only the synth module."""
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
import synth  # noqa: E402


def digests():
    out = {}
    tiny = synth.WORKLOADS["tiny"]
    c, s = synth.experts(tiny)
    out["tiny/codes"] = hashlib.sha256(c.tobytes()).hexdigest()
    out["tiny/scales"] = hashlib.sha256(s.tobytes()).hexdigest()
    out["tiny/router_w"] = hashlib.sha256(synth.router_w(tiny).tobytes()).hexdigest()
    out["tiny/x0"] = hashlib.sha256(synth.tokens_f32(tiny, [0]).tobytes()).hexdigest()
    dec = synth.WORKLOADS["decode"]
    c, s = synth.expert(dec, 0)
    out["k3/expert0/codes_first_1MiB"] = hashlib.sha256(c[:1 << 20].tobytes()).hexdigest()
    out["k3/expert0/scales"] = hashlib.sha256(s.tobytes()).hexdigest()
    out["k3/x0_bf16"] = hashlib.sha256(synth.tokens_bf16_bits(dec, [0]).tobytes()).hexdigest()
    out["k3/zipf_bias"] = hashlib.sha256(synth.router_bias(synth.WORKLOADS["decode64_zipf"]).tobytes()).hexdigest()
    out["k3/gamma_layer5"] = hashlib.sha256(synth.gamma(synth.WORKLOADS["stack12"], 5).tobytes()).hexdigest()
    return out


if __name__ == "__main__":
    with open(os.path.join(HERE, "synth_sha256.json"), "w") as f:
        json.dump(digests(), f, indent=1, sort_keys=True)
        f.write("\n")
