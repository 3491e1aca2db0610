"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds tests/sanitize/abi_host_check.cpp against the library's objects, with
csrc/moe_abi.hip (argument validation, workspace carving, queries, the launch
sequences) compiled with its host code instrumented (device code is not), and
runs it: every entry point's host-side paths that return before a launch --
workspace sizing over valid, invalid and overflowing dims, the plan-layout
query, each validation error, status strings. A sanitizer report, or a status
other than the expected one, fails the test. Host-only: skipped where a GPU is
visible, since the checks pass placeholder device pointers.
"""
import os
import shlex
import shutil
import subprocess

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_layer_gate_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "sanitize", "abi_host_check.cpp")
OTHERS = ["route.hip", "dispatch.hip", "ffn.hip", "combine.hip", "backward.hip", "probes.hip"]
# host code only: each sanitizer flag applies to the host compilation
SANITIZE = shlex.split("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                       "-Xarch_host -fno-sanitize-recover=undefined -Xarch_host -fno-omit-frame-pointer")
BASE = ["--offload-arch=gfx950", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="host-only checks with placeholder device pointers")
@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
@pytest.mark.timeout(600)
def test_abi_host_code_under_sanitizers(tmp_path):
    hipcc = _hipcc()

    def run(cmd):
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stderr[-3000:]}"

    objs = [str(tmp_path / "moe_abi_san.o")]
    procs = [subprocess.Popen([hipcc, *BASE, "-O1", "-g", *SANITIZE, "-c", os.path.join(CSRC, "moe_abi.hip"),
                               "-o", objs[0]], stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)]
    for src in OTHERS:
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen([hipcc, *BASE, "-O3", "-c", os.path.join(CSRC, src), "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    for p in procs:
        _, err = p.communicate()
        assert p.returncode == 0, err[-3000:]
    exe = str(tmp_path / "abi_host_check")
    drv = str(tmp_path / "abi_host_check.o")
    run([hipcc, *BASE, "-O1", "-g", *SANITIZE, "-c", DRIVER, "-o", drv])
    run([hipcc, "--offload-arch=gfx950", *SANITIZE, drv, *objs, "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert "all host-side ABI checks passed" in out, out[-2000:]
