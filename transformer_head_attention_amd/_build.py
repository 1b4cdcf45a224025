"""Build libmha.so (the C-ABI library) for gfx950 with hipcc, in-tree.

Every source is compiled on its own (in parallel) into ``_build/`` and the
objects are linked into ``transformer_head_attention_amd/libmha.so``.
Packed-fp32 instruction selection is disabled for all device code.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build", "libmha")
LIB = os.path.join(PKG, "libmha.so")

SOURCES = ["mha_api.hip", "prep.hip", "gemm16.hip", "attn16.hip", "fp32_path.hip", "decode.hip",
           "weights.hip", "gate.hip"]

# Per-source extra flags. The attention and decode kernels keep their MFMA
# accumulators in ordinary VGPRs (no AGPR copies around the softmax; the d_k =
# 128 decode kernel drops from 309 to 239 registers). The GEMMs are left to
# the compiler's choice (their 128 accumulators per lane fit the VGPRs).
_VGPR_MFMA = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
EXTRA = {"attn16.hip": _VGPR_MFMA, "decode.hip": _VGPR_MFMA}

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmha.so)")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass reports that it does not know the packed-fp32 feature; harmless
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + out)
    return out


def build(jobs: int = 8, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(cmds)))) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
