"""The C-ABI front end under AddressSanitizer and UBSan (CPU only).

Builds the library's sources with both sanitizers on the host side (the
device side compiled without optimisation, only so the objects link) into
one executable with tests/asan/abi_checks.cpp, and runs it.  The driver
calls every entry point with arguments the host checks must reject, and --
on a machine without a GPU -- calls that pass them and fail at their first
launch with DFLASH_ERR_HIP.  A sanitizer report or a wrong status fails.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from conftest import gpu_available

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_diffusion_drafter_concat_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

pytestmark = [
    pytest.mark.slow,
    pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available"),
    pytest.mark.skipif(gpu_available(), reason="the no-device calls pass fake device addresses"),
]

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr[-4000:]}"


def test_abi_checks_under_host_sanitizers(tmp_path):
    common = ["--offload-arch=gfx950", "-O1", "-Xarch_device", "-O0", "-std=c++17", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-I", os.path.join(ROOT, "include")] + SAN
    jobs = [[HIPCC, *common, "-c", os.path.join(CSRC, f"{s}.hip"), "-o", str(tmp_path / f"{s}.o")]
            for s in ("api", "k_small", "k_attn", "k_sample")]
    jobs.append([HIPCC, "-O1", "-std=c++17", "-I", os.path.join(ROOT, "include"), *SAN, "-x", "c++",
                 "-c", os.path.join(ROOT, "tests", "asan", "abi_checks.cpp"),
                 "-o", str(tmp_path / "drv.o")])
    with ThreadPoolExecutor(len(jobs)) as ex:
        list(ex.map(_run, jobs))
    exe = str(tmp_path / "abi_checks")
    _run([HIPCC, "--offload-arch=gfx950", *SAN[:4], "-o", exe,
          *[str(tmp_path / f"{s}.o") for s in ("drv", "api", "k_small", "k_attn", "k_sample")]])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe, "--no-device"], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    assert "abi checks ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    shutil.rmtree(tmp_path, ignore_errors=True)
