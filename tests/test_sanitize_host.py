"""The C ABI's host layer (argument validation, workspace arithmetic, the
host arrays of row splits and factors, error messages) under
AddressSanitizer and UndefinedBehaviorSanitizer.

api.hip is compiled for the host only with both sanitizers and linked,
together with the driver tests/abi_sanitize.cpp, ahead of libsg.so (whose
other host code it calls for the workspace sizes); the driver makes every
call fail validation or stop at the device check, so no kernel runs and no
GPU is needed.  Every sanitizer flag is passed to the host side only.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "post_pruning_amd")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

pytestmark = pytest.mark.skipif(
    not (os.path.exists(HIPCC) and os.path.exists(os.path.join(LIBDIR, "libsg.so"))),
    reason="hipcc or libsg.so missing")

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"
    return res


def test_abi_host_layer_sanitized(tmp_path):
    inc = "-I" + os.path.join(ROOT, "include")
    api_o, drv_o, exe = str(tmp_path / "api.o"), str(tmp_path / "drv.o"), str(tmp_path / "drv")
    _run([HIPCC, "-std=c++17", "-O1", "-g", "--offload-arch=gfx950", "--offload-host-only", "-fPIC", *SAN,
          inc, "-c", os.path.join(LIBDIR, "csrc", "api.hip"), "-o", api_o])
    _run([HIPCC, "-std=c++17", "-O1", "-g", *SAN, inc, "-x", "c++",
          os.path.join(ROOT, "tests", "abi_sanitize.cpp"), "-c", "-o", drv_o])
    _run([HIPCC, *SAN, drv_o, api_o, "-L" + LIBDIR, "-lsg", "-Wl,-rpath," + LIBDIR, "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    res = _run([exe], env=env, timeout=120)
    assert "abi host checks passed" in res.stdout
