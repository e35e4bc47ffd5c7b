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
    build_c_check(verbose)
    return out


def build_c_check(verbose: bool = False) -> str:
    """Compile tests/c_abi_check.c, a plain-C user of libdg.so, with gcc into
    c_abi_check next to the library (found there through its rpath)."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    out = os.path.join(HERE, "c_abi_check")
    src = os.path.join(os.path.dirname(HERE), "tests", "c_abi_check.c")
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(os.path.dirname(HERE), "include"), "-I", os.path.join(rocm, "include"),
           src, "-o", out + ".tmp", "-L", HERE, "-ldg", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-lm", "-Wl,-rpath,$ORIGIN", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"gcc failed on {src} ({res.returncode}):\n{res.stdout}{res.stderr}")
    if verbose and (res.stdout + res.stderr).strip():
        print(res.stdout + res.stderr, file=sys.stderr)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
