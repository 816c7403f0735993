"""Build libmoeq.so (HIP kernels for gfx950 + host packers + C ABI) in-tree.

    python -m bit_quantized_moe_route_amd.build

Device code is compiled with hipcc for gfx950 only, with packed-fp32
instruction generation disabled; host-only C++ is compiled with g++.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoeq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I", INCLUDE, "-I", CSRC,
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]


def sources():
    hip = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    cpp = sorted(f for f in os.listdir(CSRC) if f.endswith(".cpp"))
    return hip, cpp


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    hip, cpp = sources()
    jobs = []
    for f in hip:
        obj = os.path.join(BUILD, f + ".o")
        jobs.append((obj, [HIPCC] + HIP_FLAGS + ["-c", os.path.join(CSRC, f), "-o", obj]))
    for f in cpp:
        obj = os.path.join(BUILD, f + ".o")
        jobs.append((obj, ["g++"] + CXX_FLAGS + ["-c", os.path.join(CSRC, f), "-o", obj]))
    workers = min(len(jobs), max(1, (os.cpu_count() or 2)))
    with ThreadPoolExecutor(workers) as ex:
        for (obj, cmd), r in zip(jobs, ex.map(lambda j: _run(j[1]), jobs)):
            if verbose:
                print(" ".join(cmd))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp]
         + [o for o, _ in jobs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
