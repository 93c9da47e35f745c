"""Build libmagi_bca.so in-tree with hipcc for gfx950.

    python -m block_causal_attention_amd.build      # or build() from Python
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmagi_bca.so")
RATES = os.path.join(PKG, "magi_rates")  # issue-rate probe program (csrc/rates.hip)
SOURCES = ["plan.cpp", "api.cpp", "qknorm_rope.hip", "ffa_fwd.hip", "ffa_bwd.hip", "scratch.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def compile_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        # no packed-fp32 VALU instructions anywhere in the device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # device code never produces or tests NaN on purpose; this drops the
        # quieting v_max before every max (infinities stay honoured)
        "-Xarch_device", "-fno-honor-nans",
        "-Wno-unused-command-line-argument",
    ]


def build_host_sanitized(out_path: str) -> str:
    """The same library with its host code under AddressSanitizer and
    UndefinedBehaviorSanitizer (device code unchanged), for the CPU tests:
    load it with the sanitizer runtime preloaded (asan_runtime())."""
    cmd = [hipcc(), *[f for f in compile_flags() if f != "-O3"], "-O1", "-g",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
           "-shared-libsan", "-shared", "-o", out_path, *[os.path.join(CSRC, s) for s in SOURCES]]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc (sanitized host) failed ({res.returncode}):\n{res.stdout}{res.stderr}")
    return out_path


def asan_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime."""
    res = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.exists(path):
        raise RuntimeError("AddressSanitizer runtime not found")
    return path


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *compile_flags(), "-shared", "-o", tmp, *[os.path.join(CSRC, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "is not a recognized feature for this target" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    # the issue-rate probe behind the kernels' ceilings (a separate program)
    cmd = [hipcc(), *compile_flags(), "-o", RATES + ".tmp", os.path.join(CSRC, "rates.hip")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on rates.hip ({res.returncode}):\n{res.stdout}{res.stderr}")
    os.replace(RATES + ".tmp", RATES)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
