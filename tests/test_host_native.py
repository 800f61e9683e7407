"""CPU tests of native host code (no GPU).

* The router's fp64 exp (persistent_latency_bound_amd/csrc/pld_math.hpp, shared by the kernel
  and this host build) against the C library's exp: at most 2 units in the last place over
  [-700, 700] and the gates' range, exact edge cases.
* The host runtime of libpld built with AddressSanitizer and UndefinedBehaviorSanitizer on the
  host code (device code is compiled as usual): sizing of every named workload equals the
  plain library's, a seeded fuzz of configuration fields runs clean (any report aborts), and
  the argument checks return PLD_E_INVALID before any device work.
"""
import ctypes
import os
import shutil
import subprocess
import tempfile

import pytest

import persistent_latency_bound_amd as pld
from synth import configs

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "persistent_latency_bound_amd", "csrc")
INC = os.path.join(ROOT, "include")


def test_exp_f64_matches_libm():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "exp_check")
        subprocess.run(["g++", "-O2", "-std=c++17", "-I", CSRC, "-o", exe, os.path.join(HERE, "native", "exp_check.cpp")],
                       check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()
    max_ulp, edges = float(out[1]), int(out[5])
    print(f"exp_f64: max {max_ulp:.3f} ulp vs libm")
    assert max_ulp <= 2.0 and edges == 1


@pytest.mark.slow
def test_host_runtime_under_asan_ubsan():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "host_check")
        cmd = [hipcc, "-O1", "-g", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
               "-packed-fp32-ops", "-I", INC,
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
               "-x", "hip", os.path.join(CSRC, "pld_kernel.hip"), "-x", "none",
               os.path.join(HERE, "native", "host_runtime_check.cpp"), "-o", exe]
        subprocess.run(cmd, check=True, capture_output=True)
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
        res = subprocess.run([exe], capture_output=True, text=True, env=env)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr
    lines = dict((l.split()[0], l.split()[1:]) for l in res.stdout.splitlines())
    assert lines["args_ok"] == ["1"]
    print(" ".join(lines["fuzz"]))
    L = pld.lib()
    for name in ("c1", "c2", "c3", "c4", "c5", "c6", "c7"):
        s = configs.LAYERS[name]
        cfg = pld.config_from_shape(s, 32768 if name == "c5" else 0)
        for n, got in zip((1, 24), lines[name]):
            assert int(got) == L.pld_workspace_bytes_for_cus(ctypes.byref(cfg), n, 256) > 0, (name, n)
