"""Build libgdn.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: ``python -m linear_attention_recurrence_step_amd.build [--resource-usage]``.
Objects go to ``_build/`` at the repository root; the library is written next
to this file, where the Python binding loads it.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgdn.so")
SOURCES = ["gdn_abi.cpp", "gdn_record.hip", "gdn_record_mfma.hip", "gdn_replay.hip", "gdn_replay_mfma.hip",
           "gqa_expand.hip", "rms_norm.hip", "gdn_prefill.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # keep the compiler from forming packed-fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# Per-source flags.  The matrix-core replay keeps its MFMA accumulators in
# ordinary VGPRs (gfx950 allows either file): it also scales them with VALU
# instructions, and one register file instead of two doubles its occupancy.
SOURCE_FLAGS = {"gdn_replay_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "gdn_record_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "gdn_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str, extra) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + SOURCE_FLAGS.get(src, []) + list(extra) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    if extra:
        sys.stderr.write(r.stderr)
    return obj


def build(resource_usage: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []
    with ThreadPoolExecutor(max_workers=min(6, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(resource_usage="--resource-usage" in sys.argv))
