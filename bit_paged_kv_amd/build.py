"""Build libnvkv.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libnvkv.so")
# per-source extra flags.  The decode and extend-attention kernels never see NaN scores (masked
# keys are -inf, unwritten scales are zeroed), so their max trees need no NaN quieting; the
# write-side kernels keep strict IEEE semantics for bit-exact quantization.  The decode file also
# holds the fused append's quantization: from input without NaN its steps produce no NaN (+-inf
# saturates through fmin and the correctly rounded division), so the flag leaves its bytes equal to
# the standalone writer's (a GPU test compares the two on inputs with +-inf).
SOURCES = {"nvkv_quant.hip": [], "nvkv_decode.hip": ["-fno-honor-nans"], "nvkv_extend.hip": [],
           "nvkv_extend_attn.hip": ["-fno-honor-nans"], "nvkv_probe.hip": [],
           "nvkv_api.cpp": []}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-fvisibility=hidden",
    # packed-fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd, verbose):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if verbose or res.returncode != 0:
        msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l)
        if msg.strip():
            print(msg)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed: " + " ".join(cmd))


def build(verbose: bool = False) -> str:
    """Compile every source into bit_paged_kv_amd/libnvkv.so; returns the library path."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src, extra in SOURCES.items():
        obj = os.path.join(objdir, src + ".o")
        _run([HIPCC, *FLAGS, *extra, "-c", "-o", obj, os.path.join(CSRC, src)], verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
