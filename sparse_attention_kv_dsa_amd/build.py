"""Build the HIP libraries in-tree with hipcc for gfx950.

    python -m sparse_attention_kv_dsa_amd.build

produces ``libdsa.so`` (the selector, include/dsa.h) and ``libdsa_calib.so``
(measurement helpers, include/dsa_calib.h) next to this file.
"""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
CSRC = os.path.join(PKG, "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-fp32 instructions are switched off for all device code.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Wall", "-Wno-unused-function", "-Wno-pass-failed",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE]

TARGETS = {
    "libdsa.so": ["dsa.hip"],
    "libdsa_calib.so": ["calib.hip"],
}


def lib_path(name: str = "libdsa.so") -> str:
    return os.path.join(PKG, name)


def build(verbose: bool = False) -> list[str]:
    built = []
    for name, srcs in TARGETS.items():
        out = lib_path(name)
        tmp = out + ".tmp"
        cmd = [HIPCC, *FLAGS, *[os.path.join(CSRC, s) for s in srcs], "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        # the host pass warns that it does not know the packed-fp32 feature
        noise = "'-packed-fp32-ops' is not a recognized feature"
        msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed for {name}:\n" + "\n".join(msgs))
        if verbose and msgs:
            print("\n".join(msgs))
        os.replace(tmp, out)
        built.append(out)
    return built


if __name__ == "__main__":
    for p in build(verbose=True):
        print("built", p)
