"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Every source of the library is compiled as usual for gfx950, with the host
pass instrumented (``-Xarch_host -fsanitize=...``; the device code is not),
and linked against a stand-in for the HIP runtime (tests/host_check/
hip_runtime_stub.cpp) instead of libamdhip64.  A driver
(tests/host_check/abi_driver.cpp) then calls every entry point of the C ABI
with fake device addresses over the shapes of the benchmarked workloads and
the edge cases of the argument checks: validation, planning, workspace
carve-up, launch-shape computation, the trace and the static-scratch lookup
all run on the CPU, where any out-of-bounds host access, leak, signed
overflow or invalid shift stops the run, and every kernel launch is checked
for a grid and block the hardware accepts.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
CSRC = ROOT / "block_speculative_decoding_dflash2_amd" / "csrc"
HOST = Path(__file__).resolve().parent / "host_check"
BUILD = ROOT / "_build" / "host_check"
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
COMMON = ["-O1", "-g", "-std=c++17", "-fPIC", f"-I{ROOT / 'include'}"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(map(str, cmd))}\n{r.stdout}\n{r.stderr}")
    return r


@pytest.fixture(scope="module")
def driver():
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("hipcc / clang++ not available")
    BUILD.mkdir(parents=True, exist_ok=True)
    jobs = []
    for src in sorted(CSRC.glob("*.hip")):
        jobs.append([HIPCC, "--offload-arch=gfx950", *COMMON, "-Xclang", "-target-feature", "-Xclang",
                     "-packed-fp32-ops", *SAN, "-c", str(src), "-o", str(BUILD / (src.stem + ".o"))])
    jobs.append([HIPCC, "-x", "hip", "--cuda-host-only", *COMMON, *SAN, "-c",
                 str(HOST / "hip_runtime_stub.cpp"), "-o", str(BUILD / "stub.o")])
    jobs.append([HIPCC, "--cuda-host-only", *COMMON, *SAN, "-c", str(HOST / "abi_driver.cpp"),
                 "-o", str(BUILD / "driver.o")])
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        list(ex.map(_run, jobs))
    exe = BUILD / "abi_driver"
    objs = [str(BUILD / (src.stem + ".o")) for src in sorted(CSRC.glob("*.hip"))]
    _run([CLANG, "-fsanitize=address", "-fsanitize=undefined", *objs, str(BUILD / "stub.o"),
          str(BUILD / "driver.o"), "-o", str(exe)])
    return exe


def test_abi_host_code_under_asan_ubsan(driver):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([str(driver)], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert "bad launches 0, failures 0" in out, out[-4000:]
