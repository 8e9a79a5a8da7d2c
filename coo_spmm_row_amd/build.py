"""Compile libsnack_coo.so in-tree for gfx950 (hipcc for the kernels, g++ for the host code)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsnack_coo.so")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # packed fp32 VALU forms stay off
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    host_o = os.path.join(BUILD, "host.o")
    dev_o = os.path.join(BUILD, "snack_coo.o")
    topo_o = os.path.join(BUILD, "topology.o")
    cmds = [
        ["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-c",
         os.path.join(CSRC, "host.cpp"), "-o", host_o],
        ["hipcc", *HIP_FLAGS, "-c", os.path.join(CSRC, "snack_coo.hip"), "-o", dev_o],
        ["hipcc", *HIP_FLAGS, "-c", os.path.join(CSRC, "topology.hip"), "-o", topo_o],
        ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", dev_o, topo_o, host_o, "-o", LIB + ".tmp"],
    ]
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"build failed: {' '.join(cmd)}\n{res.stdout[-4000:]}\n{res.stderr[-4000:]}")
        err = "\n".join(ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln
                        and "target-feature" not in ln)
        if verbose and err.strip():
            print(err)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
