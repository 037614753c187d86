"""Build the test-only probe library tests/probe/libmfma_probe.so (hipcc, gfx950)."""

from __future__ import annotations

import os
import subprocess

from moe_expert_layer_sigmoid_amd import build as libbuild

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libmfma_probe.so")


def build() -> str:
    tmp = LIB + ".tmp"
    cmd = [libbuild.hipcc(), f"--offload-arch={libbuild.ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(HERE, "mfma_probe.hip"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on mfma_probe.hip:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
