"""Build libdg.so in-tree with hipcc for gfx950 (MI355X)."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = ["dg_api.hip", "k_gemm.hip", "k_attn.hip", "k_logits.hip", "k_selfcond.hip",
           "k_sampler.hip", "k_moe.hip", "k_peak.hip"]
# Packed fp32 VALU forms are disabled for all device code.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    out = os.path.join(HERE, "libdg.so")
    tmp = out + ".tmp"
    srcs = [os.path.join(HERE, "csrc", s) for s in SOURCES]
    cmd = [hipcc()] + FLAGS + ["-o", tmp] + srcs
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msg}")
    if verbose and msg.strip():
        print(msg, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
