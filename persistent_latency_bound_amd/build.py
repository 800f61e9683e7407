"""Build the HIP libraries in-tree for gfx950 (hipcc; cross-compiles without a GPU).

    python -m persistent_latency_bound_amd.build

Outputs:
  persistent_latency_bound_amd/libpld.so   the decode library (C ABI in include/pld.h)
  synth/libsynth_gen.so                    the device half of the seeded input generator
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "persistent_latency_bound_amd")
ARCH = os.environ.get("PLD_OFFLOAD_ARCH", "gfx950")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    # packed fp32 instructions stay off (hipcc's host pass warns that it does not know the feature)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]

TARGETS = [
    (os.path.join(PKG, "csrc", "pld_kernel.hip"), os.path.join(PKG, "libpld.so"),
     ["-I", os.path.join(ROOT, "include")]),
    (os.path.join(ROOT, "synth", "csrc", "synth_gen.hip"), os.path.join(ROOT, "synth", "libsynth_gen.so"),
     ["-ffp-contract=off"]),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> None:
    cc = hipcc()
    for src, out, extra in TARGETS:
        tmp = out + ".tmp"
        cmd = [cc, *COMMON, *extra, "-o", tmp, src]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"hipcc failed for {src}")
        os.replace(tmp, out)


if __name__ == "__main__":
    build(verbose=True)
    print("built")
