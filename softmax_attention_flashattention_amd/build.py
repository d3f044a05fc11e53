"""Builds libattn.so (HIP, gfx950) in this package directory.

Usage: ``python -m softmax_attention_flashattention_amd.build``.  The library
is one translation unit compiled with hipcc for gfx950 only.  Packed fp32
VALU instructions are disabled (``-packed-fp32-ops``); hipcc's host pass warns
that it does not know that feature, which is harmless.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "attn_api.hip")
OUT = os.path.join(PKG, "libattn.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(PKG, "csrc"),
]


def build(verbose=False, extra_flags=()):
    """Compiles libattn.so; returns its path.  Raises on a compile error."""
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    tmp = OUT + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, *extra_flags, SRC, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if verbose or res.returncode != 0:
        noise = "is not a recognized feature for this target"
        msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
        if msg:
            print(msg, file=sys.stderr)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed building libattn.so")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
