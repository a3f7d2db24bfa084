"""Build libstrata_moe.so (the layer) and libstrata_probe.so (matrix-unit
measurements for the benchmark and tests) in-tree with hipcc for gfx950.

Every source compiles to its own object (in parallel), then hipcc links each
shared library next to this file.  Flags:
  --offload-arch=gfx950          the only target
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                 no packed fp32 instructions (the host pass
                                 warns that it does not know the feature)
  -fhip-fp32-correctly-rounded-divide-sqrt
                                 IEEE fp32 division (the int8 rounding of the
                                 activations depends on it)
  -mllvm -amdgpu-mfma-vgpr-form  MFMA results in VGPRs: the block loop reads
                                 every result with VALU FMAs
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libstrata_moe.so")
SOURCES = ["strata_moe.hip", "k_quant.hip", "k_route.hip", "k_group.hip", "k_experts.hip", "k_gemv.hip",
           "k_pack.hip"]
PROBE_LIB = os.path.join(HERE, "libstrata_probe.so")
PROBE_SOURCES = ["probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall",
    "-Wno-unused-function",
]


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def _link(objs: list, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link both libraries; returns the layer
    library's path."""
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as pool:
        objs = dict(zip(srcs, pool.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
