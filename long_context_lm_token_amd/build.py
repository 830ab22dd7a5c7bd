"""Build the gfx950 HIP library libttt.so in-tree with hipcc.

Usage: python -m long_context_lm_token_amd.build   (or build() from Python)
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libttt.so")
SOURCES = ["gemm.hip", "attention.hip", "elementwise.hip", "runtime.cpp", "kapi.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 VALU ops (v_pk_*_f32) in any HIP code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def _compile(hipcc: str, src: str) -> str:
    obj = os.path.join(HERE, "_build", src + ".o")
    cmd = [hipcc] + [f for f in HIPCC_FLAGS if f != "-shared"] + ["-x", "hip", "-c",
                                                                     os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(os.path.join(HERE, "_build"), exist_ok=True)
    # one hipcc per source, in parallel (each is a separate process)
    jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", "0")) or (os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(hipcc, s), SOURCES))
    if verbose:
        for o in objs:
            print("built", o)
    tmp = LIB + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
