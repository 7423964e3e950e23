"""Build libmoe_mxfp4.so for gfx950 with hipcc (in-tree): each source to an
object in parallel, then one link."""
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_mxfp4.so")
SOURCES = ["abi.hip", "route.hip", "expert_gemv.hip", "expert_mfma.hip", "misc.hip", "residency.hip", "route_trace.hip", "int8_gemv.hip", "mfma_rate.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions, no fast-math, IEEE denormals
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-fast-math", "-ffp-contract=fast-honor-pragmas",
    "-Wall", "-Wno-unused-function",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    return r.returncode, out


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    objdir = tempfile.mkdtemp(prefix="moe_build_")
    try:
        objs = [os.path.join(objdir, os.path.basename(s) + ".o") for s in srcs]
        cmds = [[HIPCC, *FLAGS, "-c", "-I", os.path.join(ROOT, "include"), "-o", o, src] for src, o in zip(srcs, objs)]
        jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
        with ThreadPoolExecutor(jobs) as pool:
            results = list(pool.map(_run, cmds))
        for cmd, (rc, out) in zip(cmds, results):
            if verbose:
                print(" ".join(cmd))
            if rc != 0:
                raise RuntimeError("hipcc failed:\n" + out)
            if out.strip() and verbose:
                print(out)
        tmp = LIB + ".tmp%d" % os.getpid()
        rc, out = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
        if rc != 0:
            raise RuntimeError("hipcc link failed:\n" + out)
        os.replace(tmp, LIB)
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
