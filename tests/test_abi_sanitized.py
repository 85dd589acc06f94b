"""The library's host code (graph checks, planning, workspace sizing, argument
validation) built with AddressSanitizer and UndefinedBehaviorSanitizer and run
through the host-only checks of tests/sanitize/abi_checks.cpp: every call
returns the expected status and the sanitizers report nothing.  The HIP kernel
objects are linked unchanged (no device code runs)."""
import os
import shutil
import subprocess

import pytest

from helpers import ROOT, ensure_built

CSRC = os.path.join(ROOT, "linear_bound_propagation_amd", "csrc")
OBJ = os.path.join(ROOT, "_build")
KERNEL_OBJS = ["vb_gemm.o", "vb_ibp_narrow.o", "vb_kernels.o", "vb_scratch.o"]


def test_host_code_under_asan_and_ubsan(tmp_path):
    ensure_built()
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no g++")
    objs = [os.path.join(OBJ, o) for o in KERNEL_OBJS]
    missing = [o for o in objs if not os.path.exists(o)]
    assert not missing, f"kernel objects missing (run the build first): {missing}"
    exe = str(tmp_path / "abi_checks")
    cmd = [gxx, "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "sanitize", "abi_checks.cpp"), os.path.join(CSRC, "vb_api.cpp")] + objs + \
          ["-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = run.stdout + run.stderr
    print(out[-3000:])
    assert run.returncode == 0, out[-3000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]
    assert "0 failure(s)" in out
