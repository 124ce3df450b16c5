"""Builds libdsa.so in-tree with hipcc for gfx950.

Each source compiles in its own process (in parallel), then hipcc links the
shared library.  Every HIP source is compiled with packed-FP32 instructions
disabled (``-Xclang -target-feature -Xclang -packed-fp32-ops``).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdsa.so")
OBJDIR = os.path.join(HERE, "_build")
SOURCES = ["api.hip", "index_scores.hip", "prefill_scores.hip", "prefill_topk.hip", "topk.hip", "attn.hip", "decode.hip", "append.hip", "recall.hip"]
# per-source extra flags: the prefill contraction and the gathered attention
# keep their MFMA results in VGPRs, which saves the accumulation-register
# reads and writes around their epilogues (the attention's online softmax
# rescales its output tiles on the VALU)
EXTRA = {"prefill_scores.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm 7 is required to build libdsa.so)")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is noise
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(OBJDIR, exist_ok=True)
    objs = [os.path.join(OBJDIR, s.replace(".hip", ".o")) for s in SOURCES]
    cmds = [[hipcc, *FLAGS, *EXTRA.get(s, []), "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    with cf.ThreadPoolExecutor(max_workers=min(9, len(cmds))) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
