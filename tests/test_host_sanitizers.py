"""The C ABI's host-side argument checks and workspace queries under
AddressSanitizer and UndefinedBehaviorSanitizer (CPU only): gdpa_api.cpp's
host code is rebuilt with both sanitizers, linked with the library's kernel
objects into tests/sanitize_driver.cpp, and run.  The driver's calls are all
refused (or empty) before anything reaches a GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "generalized_attention_amd", "csrc")
OBJDIR = os.path.join(ROOT, "generalized_attention_amd", "_build")
HIPCC = "/opt/rocm/bin/hipcc"


@pytest.mark.timeout(600)
def test_argument_checks_under_asan_and_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc is not installed")
    kernels = [os.path.join(OBJDIR, f) for f in sorted(os.listdir(OBJDIR))
               if f.endswith(".o") and f != "gdpa_api.o"] if os.path.isdir(OBJDIR) else []
    if not kernels:
        subprocess.run(["python3", os.path.join(ROOT, "generalized_attention_amd", "build.py")], check=True)
        kernels = [os.path.join(OBJDIR, f) for f in sorted(os.listdir(OBJDIR)) if f.endswith(".o") and f != "gdpa_api.o"]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    api = str(tmp_path / "api.o")
    subprocess.run([HIPCC, "-x", "hip", "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
                    *san, "-c", os.path.join(CSRC, "gdpa_api.cpp"), "-o", api], check=True, capture_output=True)
    drv = str(tmp_path / "driver.o")
    subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
                    "-c", os.path.join(ROOT, "tests", "sanitize_driver.cpp"), "-o", drv], check=True,
                   capture_output=True)
    exe = str(tmp_path / "driver")
    # kernel objects only hold device code and its registration; only the
    # host code under test is instrumented
    subprocess.run([HIPCC, "--offload-arch=gfx950", *san, drv, api, *kernels, "-o", exe], check=True,
                   capture_output=True)
    # no GPU is visible to the driver: a call that passed the checks by
    # mistake fails in the runtime instead of launching a kernel
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="", ROCR_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "ok" in r.stdout, r.stdout[-4000:] + r.stderr[-4000:]
