"""Build libscfa.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Each translation unit is compiled to an object in ``_build/`` (in parallel),
then linked into ``sparse_causal_attention_amd/libscfa.so``.  Runs on a
machine without a GPU: hipcc cross-compiles for the target architecture.
"""

from __future__ import annotations

import concurrent.futures
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libscfa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["api.cpp", "meta.hip", "attn_fwd.hip", "attn_bwd.hip", "lsh.hip", "rows.hip", "noalloc.hip"]

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed fp32 VALU forms are kept out of the generated code on purpose
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core results go straight to VGPRs (no AGPR copies around the softmax)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


# Kernels the benchmark times (d = 64, block 64: the bf16 attention kernels reading rows through the sort
# permutations in the pruned modes, the dense-causal baseline over plain rows, the stored-dS backward).  Each
# must compile without scratch (register spills); the build fails otherwise.
NO_SCRATCH = [
    r"k_fwd_bf16_ksILi[12]ELi64ELi64ELb1E", r"k_fwd_bf16_ksILi0ELi64ELi64ELb0E",
    r"k_bwd_dq_bf16ILi[12]ELi64ELi64ELb1E", r"k_bwd_dq_bf16ILi0ELi64ELi64ELb0E",
    r"k_bwd_dkdv_bf16ILi[12]ELi64ELi64ELb1E", r"k_bwd_dkdv_bf16ILi0ELi64ELi64ELb0E",
    r"k_bwd_dq_ds_bf16ILi64ELi64E",
]


def _scratch_by_kernel(remarks: str) -> dict:
    """{mangled kernel name: scratch bytes per lane} from -Rpass-analysis=kernel-resource-usage remarks."""
    out, cur = {}, None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and cur:
            out[cur] = int(m.group(1))
    return out


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.startswith("attn_"):
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    if src.startswith("attn_"):
        spills = {k: v for k, v in _scratch_by_kernel(r.stderr).items()
                  if v > 0 and any(re.search(p, k) for p in NO_SCRATCH)}
        if spills:
            raise RuntimeError(f"timed kernels in {src} use scratch (register spills): {spills}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    workers = min(len(SOURCES), max(1, len(os.sched_getaffinity(0))))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
