"""Build libgdn.so (gfx950) in-tree with hipcc.

    python gated_deltanet_recurrent_chunk_amd/build.py [--verbose]

(run by path: importing the package loads the library this script builds)

Objects go to gated_deltanet_recurrent_chunk_amd/_build/, the library to
gated_deltanet_recurrent_chunk_amd/libgdn.so.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgdn.so")
ROOT = os.path.dirname(HERE)

SOURCES = ["plan.cpp", "gdn_api.cpp", "prefill_kernels.hip", "flush_kernel.hip", "stream_kernels.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-I", os.path.join(ROOT, "include"),
          "-Wall", "-Wno-unused-function",
          # no packed fp32 instructions in device code
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # matrix-core results in ordinary VGPRs: the kernels read every product back
          # with vector instructions, and accumulators in AGPRs cost a copy per register
          "-mllvm", "-amdgpu-mfma-vgpr-form"]
# per-source flags: the flush kernel takes its two per-request index arrays as leading
# scalar arguments, preloaded into SGPRs at wave launch (one memory round trip fewer
# before its first loads)
EXTRA = {"flush_kernel.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=4"]}


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.rsplit(".", 1)[0] + ".o")
        objs.append(obj)
        cmd = [HIPCC] + COMMON + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".hip"):
            cmd = cmd[:1] + ["-x", "hip"] + cmd[1:]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        # the host pass does not know the device-only target feature: harmless
        lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l]
        if lines and (verbose or p.returncode != 0):
            print("\n".join(lines), flush=True)
        if p.returncode != 0:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="--verbose" in sys.argv)
    print(LIB)
