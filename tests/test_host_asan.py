"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds vc_api.hip (argument checks, workspace layout, launch plan) with
asan/launch_stubs.cpp and asan/abi_checks.cpp, the host pass instrumented by
-fsanitize=address,undefined (the device pass stays as it is), and runs the
driver: every rejection path of every entry point, layouts from one token to
the largest supported shapes, the per-thread last error.  Calls that pass
every check end in host stand-ins of the kernel launchers, so nothing runs on
a GPU and no GPU is needed.  Any sanitizer report, leak included, fails the
run.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_abi_checks_under_host_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_checks")
    cmd = [HIPCC, "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "bit_attention_video_vc_amd", "csrc"),
           os.path.join(ROOT, "bit_attention_video_vc_amd", "csrc", "vc_api.hip"),
           os.path.join(ROOT, "tests", "asan", "launch_stubs.cpp"),
           os.path.join(ROOT, "tests", "asan", "abi_checks.cpp"),
           "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert b.returncode == 0, b.stderr[-4000:]
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["HIP_VISIBLE_DEVICES"] = ""  # the driver never needs a device
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert "Sanitizer" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    last = [ln for ln in r.stdout.splitlines() if ln.startswith("abi_checks:")]
    assert last and last[0].endswith(" 0 failures"), out[-6000:]
    n = int(last[0].split()[1])
    assert n >= 80, last[0]
