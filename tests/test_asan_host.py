"""The library's host code (argument validation, size functions, the I2V
mask helper) under AddressSanitizer: every HIP source is rebuilt with the
sanitizer on the host side only, linked into tests/asan/abi_validate.cpp,
and run on the CPU.  Every call the driver makes fails validation or touches
host memory only, so no GPU is needed."""
import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "video_diffusion_transformer_block_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
OUT = os.path.join(ROOT, "_build", "asan")
# the sanitizer applies to the host compilation only (-Xarch_host before each option)
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
         "-Xclang", "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include")] + HOST_ASAN


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_host_validation_under_asan():
    os.makedirs(OUT, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(OUT, os.path.basename(s) + ".o") for s in srcs]
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        list(ex.map(lambda so: _run([HIPCC, *FLAGS, "-c", so[0], "-o", so[1]]), zip(srcs, objs)))
    # the driver is plain host C++: g++ with the sanitizer, and g++ links it with
    # the sanitized objects and the HIP runtime
    drv = os.path.join(OUT, "abi_validate.o")
    _run(["g++", "-O1", "-g", "-fsanitize=address", "-fno-omit-frame-pointer",
          "-I" + os.path.join(ROOT, "include"), "-c", os.path.join(ROOT, "tests", "asan", "abi_validate.cpp"),
          "-o", drv])
    exe = os.path.join(OUT, "abi_validate")
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(HIPCC)))
    _run(["g++", "-fsanitize=address", drv, *objs, "-L" + os.path.join(rocm, "lib"), "-lamdhip64",
          "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and "OK" in r.stdout, f"{r.stdout}\n{r.stderr[-4000:]}"
