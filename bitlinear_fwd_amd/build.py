"""Build libbitlinear.so in-tree with hipcc for gfx950 (MI355X).

    python -m bitlinear_fwd_amd.build          # compile every HIP source, link the library
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libbitlinear.so")
SOURCES = ["bitlinear_api.hip", "weight_quant.hip", "act_quant.hip", "gemv.hip", "gemv_lut.hip", "gemv_bin.hip",
           "gemm.hip", "probes.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no FMA contraction, no fast-math: the quantisers' roundings are part of the contract
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # keep the compiler from forming packed fp32 ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile the sources to objects (in parallel, at most `jobs` at once; 0 = one per
    CPU up to 8), then link the shared library atomically."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 1)
    objs, procs, pending = [], [], list(SOURCES)
    while pending or procs:
        while pending and len(procs) < jobs:
            src = pending.pop(0)
            obj = os.path.join(objdir, src.replace(".hip", ".o"))
            cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
        src, proc = procs.pop(0)
        out, _ = proc.communicate()
        if proc.returncode != 0:
            sys.stderr.write(out)
            for _, other in procs:
                other.wait()
            raise RuntimeError(f"hipcc failed on {src}")
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("link of libbitlinear.so failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
