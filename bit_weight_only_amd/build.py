"""Build libnf4.so (hand-written HIP for gfx950) in-tree with hipcc.

    python -m bit_weight_only_amd.build

Every source is compiled for gfx950 only, with packed-fp32 instruction
selection switched off, then linked into ``bit_weight_only_amd/libnf4.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libnf4.so")
BUILD = os.path.join(ROOT, "_build")

SOURCES = ["nf4_abi.hip", "pack.hip", "gemv.hip", "gemm.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-instruction results in VGPRs: the compiler otherwise picks the
    # AGPR form for kernels that may use more than 256 registers, and every
    # product read by a vector instruction then costs v_accvgpr_read moves
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include"),
]


# the compiler's per-kernel resource report, read to refuse register spills
REPORT = "-Rpass-analysis=kernel-resource-usage"


def scratch_kernels(report: str) -> list[tuple[str, int]]:
    """(kernel, bytes per lane) for every kernel of a resource report whose
    private segment is nonzero, i.e. that spills registers to scratch."""
    out, name = [], None
    for ln in report.splitlines():
        m = re.search(r"Function Name: (\S+)", ln)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", ln)
        if m and int(m.group(1)) > 0:
            out.append((name, int(m.group(1))))
    return out


# Per-source flags.  gemv.hip: the decode kernels' first eight arguments
# (the fast GEMV puts the ones its first weight loads need there) arrive in
# scalar registers at dispatch instead of through reads of the argument
# memory; firmware without that feature runs the loads the compiler places
# at the kernel's entry for it.  And the instruction scheduler that favours
# instruction-level parallelism: the decode step of 113 launches took
# 1.106 -> 1.080 ms at M = 1 and 1.185 -> 1.160 ms at M = 2 with it (the
# same instructions, reordered; the memory-clause scheduler was no faster).
SOURCE_FLAGS = {"gemv.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=8",
                             "-mllvm", "-amdgpu-sched-strategy=max-ilp"]}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), REPORT, "-c", os.path.join(CSRC, src),
           "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    spills = scratch_kernels(r.stderr)
    if spills:
        raise RuntimeError(f"{src}: kernels spill registers to scratch (bytes per lane):\n" +
                           "\n".join(f"  {b:5d}  {k}" for k, b in spills))
    # hipcc's host pass does not know the packed-fp32 feature; that warning is harmless
    noise = [ln for ln in r.stderr.splitlines() if ("warning" in ln or "error" in ln)
             and "packed-fp32-ops" not in ln and "not a recognized feature" not in ln]
    if verbose and noise:
        print("\n".join(noise), file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
