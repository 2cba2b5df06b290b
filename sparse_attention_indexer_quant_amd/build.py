"""Build libdsaidx.so in-tree with hipcc for gfx950.

    python -m sparse_attention_indexer_quant_amd.build

Every HIP source is compiled with -ffp-contract=off (the quantizers' bytes depend on each
float operation being a single IEEE operation) and without packed-FP32 instructions.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIBRARY = os.path.join(HERE, "libdsaidx.so")
ARCH = "gfx950"


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")
    return path


def common_flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
            "-fhip-fp32-correctly-rounded-divide-sqrt",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # matrix results land in VGPRs, read directly by the epilogue
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            # the leading kernel arguments arrive in scalar registers at wave launch instead of
            # being loaded from memory (the code object keeps a fallback that loads them)
            "-mllvm", "-amdgpu-kernarg-preload-count=16",
            "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]


def kernel_resources(remarks: str) -> dict[str, dict[str, str]]:
    """Per-kernel resource lines of hipcc's kernel-resource-usage remarks."""
    out: dict[str, dict[str, str]] = {}
    name = None
    for line in remarks.splitlines():
        if "remark:" not in line or "kernel-resource-usage" not in line:
            continue
        text = line.split("remark:", 1)[1].rsplit("[-Rpass", 1)[0].strip()
        key, _, val = text.partition(":")
        if key == "Function Name":
            name = val.strip()
            out[name] = {}
        elif name is not None:
            out[name][key.strip()] = val.strip()
    return out


def _compile(src: str) -> str:
    """Compile one source; a kernel that spills to scratch memory fails the build (scratch
    setup slows every wave launch, and a spill in a hot loop costs a memory round trip)."""
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc()] + common_flags() + ["-Rpass-analysis=kernel-resource-usage", "-c", src,
                                        "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{proc.stderr}")
    for kernel, res in kernel_resources(proc.stderr).items():
        if res.get("ScratchSize [bytes/lane]", "0") != "0":
            raise RuntimeError(f"{src}: kernel {kernel} uses scratch memory: {res}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libdsaidx.so (always rebuilds)."""
    os.makedirs(BUILD, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "capi.cpp")]
    workers = min(len(sources), max(1, (os.cpu_count() or 4) // 2), 8)
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(_compile, sources))
    tmp = LIBRARY + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"link failed:\n{proc.stderr}")
    os.replace(tmp, LIBRARY)
    if verbose:
        print(f"built {LIBRARY}")
    return LIBRARY


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
