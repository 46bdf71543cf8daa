"""The C-ABI's argument validation under AddressSanitizer and UndefinedBehaviorSanitizer.

tp_api.hip and the launch planner (gemm_plan.hip) are compiled with the sanitizers on the
host side and linked with stub launchers (tests/sanitize/launch_stubs.cpp) and a driver
(tests/sanitize/validate_main.cpp) that calls every entry point with documented invalid
arguments and with sweeps of extreme sizes; any sanitizer report, or a status outside the
documented set, fails the test.  No kernel is launched: the stubs return an error.
"""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT, gpu_available

pytestmark = pytest.mark.skipif(gpu_available(), reason="host-only sanitizer build")

CSRC = os.path.join(ROOT, "megatron_tensor_transformer_linear_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")


def hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    pytest.skip("hipcc not found")


def test_validation_is_clean_under_asan_and_ubsan(tmp_path):
    cc = hipcc()
    # sanitizers on the host side only (-Xarch_host before each); device code stays as built
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Wno-inline-asm",
              "-I" + os.path.join(ROOT, "include"),
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + san
    objs = []
    for src, lang in ((os.path.join(CSRC, "tp_api.hip"), None),
                      (os.path.join(CSRC, "gemm_plan.hip"), None),
                      (os.path.join(SAN, "launch_stubs.cpp"), "hip"),
                      (os.path.join(SAN, "validate_main.cpp"), "c++")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        cmd = [cc] + common + (["-x", lang] if lang else []) + ["-c", src, "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stdout + res.stderr
        objs.append(obj)
    exe = str(tmp_path / "validate")
    res = subprocess.run([cc, "--offload-arch=gfx950"] + san + objs + ["-o", exe],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert " 0 failures" in out
