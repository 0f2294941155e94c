"""Build libawq.so in-tree with hipcc for gfx950.

    python -m weight_only_bit_w4a16_amd.build        # or build() from Python

Every HIP source under csrc/ is compiled to an object under _build/ (in
parallel) and linked into weight_only_bit_w4a16_amd/libawq.so. The
measurement probes of the benchmark (csrc/probe/) go into a library of their
own, libawq_probe.so, outside the product's ABI.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libawq.so")
PROBE_SRC = os.path.join(CSRC, "probe", "k_probe.hip")
PROBE_LIB = os.path.join(PKG, "libawq_probe.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

# -ffp-contract=off: the quantizer's float32 steps must be single roundings
# (no silent FMA contraction); FMAs are written explicitly where wanted.
# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# per-source extra flags: the decode kernels keep their MFMA results in
# VGPRs (they are read back right away), the prefill kernel in AGPRs
EXTRA = {
    "k_gemv.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"],
    "k_gemv_mb.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"],
}


def sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    path = src if os.path.isabs(src) else os.path.join(CSRC, src)
    cmd = [HIPCC, *COMMON, *EXTRA.get(src, []), "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs + [PROBE_SRC]))
    probe_obj = objs.pop()
    for lib, o in ((LIB, objs), (PROBE_LIB, [probe_obj])):
        tmp = lib + ".tmp"
        cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *o, "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        os.replace(tmp, lib)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
