"""Build libprkv.so in-tree for gfx950.

    python -m pre_rope_kv_amd.build        (or __graft_entry__.build())

The host half (prkv_host.cpp) is plain C++17 built with g++; the device half
(prkv_inject.hip, prkv_retrieve.hip, prkv_attend.hip) is built with hipcc for
gfx950 only.  libprkv_ceiling.so (prkv_ceiling.hip: a plain copy, a streaming read and a
gather of the attention launch's cache rows) is built beside it for the
bench's attainable-bandwidth references.  Packed fp32 VALU
instructions are disabled and FP contraction is off: the compensated
rotation relies on every product and sum being rounded exactly as written.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libprkv.so")
# bench-only: a plain streaming copy with the inject kernel's memory
# instructions, the attainable-bandwidth reference the bench reports
CEILING_LIB = os.path.join(HERE, "libprkv_ceiling.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"
DEVICE_SOURCES = ["prkv_inject.hip", "prkv_retrieve.hip", "prkv_attend.hip"]

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd[:2])} ... (exit {res.returncode})")
    return res


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    host_o = os.path.join(BUILD, "prkv_host.o")
    _run(["g++", "-std=c++17", "-O2", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE,
          "-c", os.path.join(CSRC, "prkv_host.cpp"), "-o", host_o], verbose)
    objs = [host_o]
    for src in DEVICE_SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        _run([hipcc, *HIP_FLAGS, "-I", INCLUDE, "-c", os.path.join(CSRC, src), "-o", obj],
             verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs,
          f"-Wl,-rpath,{ROCM}/lib"], verbose)
    os.replace(tmp, LIB)
    ceil_o = os.path.join(BUILD, "prkv_ceiling.o")
    _run([hipcc, *HIP_FLAGS, "-c", os.path.join(CSRC, "prkv_ceiling.hip"), "-o", ceil_o], verbose)
    tmp = CEILING_LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, ceil_o,
          f"-Wl,-rpath,{ROCM}/lib"], verbose)
    os.replace(tmp, CEILING_LIB)
    return LIB


def device_asm(out_path, source="prkv_inject.hip"):
    """Write the gfx950 assembly of one device source (for inspection only)."""
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    _run([hipcc, *HIP_FLAGS, "-I", INCLUDE, "--cuda-device-only", "-S",
          os.path.join(CSRC, source), "-o", out_path], False)


if __name__ == "__main__":
    print(build(verbose=True))
