"""The host half of the library under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

pool.cpp, plan.cpp, api.cpp and caps.cpp -- the fork bookkeeping, eviction and refill, the
decode planner with its in-place rebuild, the batched append and the argument checks of the
entry points -- are compiled with -fsanitize=address,undefined into one program with
tests/sanitize_driver.c, a randomized client of the C header, and the device launchers
stubbed (tests/sanitize_stubs.cpp: no kernels are built or run).  Any sanitizer report, leak
or violated bookkeeping check fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "lora_shared_prefix_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if shutil.which("g++") is None or shutil.which("gcc") is None:
        pytest.skip("no host compiler")
    if not os.path.isdir(os.path.join(ROCM, "include", "hip")):
        pytest.skip("no HIP headers")
    out = tmp_path_factory.mktemp("san")
    inc = ["-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROCM, "include"), "-I" + CSRC]
    objs = []
    for src in ("pool.cpp", "plan.cpp", "api.cpp", "caps.cpp"):
        obj = str(out / (src + ".o"))
        subprocess.run(["g++", "-std=c++17", *SAN, *inc, "-c", os.path.join(CSRC, src), "-o",
                        obj], check=True, capture_output=True, text=True, timeout=300)
        objs.append(obj)
    obj = str(out / "stubs.o")
    subprocess.run(["g++", "-std=c++17", *SAN, *inc, "-c",
                    os.path.join(ROOT, "tests", "sanitize_stubs.cpp"), "-o", obj],
                   check=True, capture_output=True, text=True, timeout=300)
    objs.append(obj)
    obj = str(out / "driver.o")
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", *SAN, *inc, "-c",
                    os.path.join(ROOT, "tests", "sanitize_driver.c"), "-o", obj],
                   check=True, capture_output=True, text=True, timeout=300)
    objs.append(obj)
    exe = str(out / "driver")
    link = subprocess.run(["g++", *SAN, *objs, "-o", exe, "-L" + os.path.join(ROCM, "lib"),
                           "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")],
                          capture_output=True, text=True, timeout=300)
    assert link.returncode == 0, link.stdout + link.stderr
    return exe


def test_host_library_is_clean_under_asan_and_ubsan(driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               LSAN_OPTIONS="suppressions=" + os.path.join(ROOT, "tests", "lsan_suppressions.txt"))
    run = subprocess.run([driver, "300"], capture_output=True, text=True, timeout=600, env=env)
    assert run.returncode == 0 and run.stdout.strip().endswith("ok"), run.stdout + run.stderr[-4000:]
    counts = dict(kv.split("=") for kv in run.stdout.strip().splitlines()[-2].split())
    print("[sanitizers]", counts)
    assert all(int(v) > 0 for v in counts.values()), counts  # every path was exercised
