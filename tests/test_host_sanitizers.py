"""AddressSanitizer and UndefinedBehaviorSanitizer on the library's host code.

The host side of every source in the library (argument validation, workspace
layout, dispatch; hipcc --cuda-host-only, so no device code is built) is
compiled with both sanitizers (relocatable device code, so the host objects
need no device binary) and linked with tests/host_abi_driver.cpp,
which calls every entry point with invalid and with valid arguments on a
machine without a GPU (calls stop at validation or at the device check; no
kernel is launched).  Any sanitizer report aborts the driver."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.abspath(os.path.dirname(__file__)))
CSRC = os.path.join(ROOT, "quantized_moe_expert_lds_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "host_abi_driver.cpp")


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
COMMON = ["-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("hostsan")
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))

    def compile_one(src):
        obj = os.path.join(out, os.path.basename(src) + ".o")
        cmd = [hipcc, *COMMON, "--offload-arch=gfx950", "-fgpu-rdc", "--cuda-host-only", *SAN, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stderr[-3000:]}"
        return obj

    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv_obj = os.path.join(out, "driver.o")
    r = subprocess.run([hipcc, *COMMON, *SAN, "-x", "c++", "-c", DRIVER, "-o", drv_obj], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = os.path.join(out, "host_abi_driver")
    r = subprocess.run([hipcc, "--offload-arch=gfx950", "-fgpu-rdc", *SAN, drv_obj, *objs, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


def test_host_code_under_asan_and_ubsan(driver):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"    # the HIP runtime keeps allocations until exit
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["HIP_VISIBLE_DEVICES"] = ""                               # never touch a device, even where one exists
    r = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, f"exit {r.returncode}\n{r.stdout[-2000:]}\n{r.stderr[-4000:]}"
    assert "host ABI driver: ok" in r.stdout
