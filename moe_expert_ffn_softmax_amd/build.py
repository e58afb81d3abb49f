"""Build libafd_ffn.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m moe_expert_ffn_softmax_amd.build
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build", "afd_ffn")
LIB = os.path.join(PKG, "libafd_ffn.so")
PROBE_LIB = os.path.join(PKG, "libafd_probe.so")  # measurement probes of bench.py --attainable
PROBE_SRC = os.path.join(CSRC, "probe", "attainable.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed-fp32 instructions are kept out of the generated code (see the project notes on
# gfx950 code generation); hipcc's host pass warns that it does not know the feature.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", INCLUDE, "-I", CSRC]


# Per-file code-generation options.  The fp8 tiled GEMM rescales every MFMA result
# with VALU FMAs; asking for the VGPR form of the MFMA destination keeps the results
# out of the accumulator registers (no copy back per value).
FILE_FLAGS = {"gemm_fp8_tiled.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def flags_for(src: str):
    return [*HIP_FLAGS, *FILE_FLAGS.get(os.path.basename(src), [])]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *flags_for(src), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(jobs: int = 0) -> str:
    """Compile every .hip source of the library and link libafd_ffn.so, and the
    measurement probes into libafd_probe.so.  Always recompiles (the caller asked for
    a build)."""
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs) + 1, max(1, min(16, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs + [PROBE_SRC]))
    _link(objs[:-1], LIB)
    _link(objs[-1:], PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build())
