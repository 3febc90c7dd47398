"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

Two drivers under tests/sanitize/ are built with gcc/g++ and -fsanitize=address,undefined
(plus float-cast-overflow, which gcc's undefined set leaves out) and -fno-sanitize-recover,
so the first report ends the run with a non-zero status:

  * kvq_api_driver.cpp links the library's host half (kvq_api.cpp: validation, buffer and
    workspace sizing, the launch plan of appends with a recent window, the split of decode
    calls, the allocation-free entry point's limit, the codebook helper) against host
    stand-ins for the launchers that write and read every byte the kernels may, on buffers
    of exactly the sizes the library reports, and checks the append plan against the packed
    layout the header states.
  * oracle_driver.c runs the oracle's encoder and attention over every key and value format
    on exact-size buffers (zero-byte ones for buffers a format does not use), with inputs at
    the ends of the fp16 domain, and checks attention's convex-hull property.

The device code is not built here: these are host builds with g++/gcc only.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "bit_kv_cache_kvq_amd", "csrc")
HIP_INCLUDE = "/opt/rocm/include"
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined,float-cast-overflow",
             "-fno-sanitize-recover=all"]


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} not installed")


def _build(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, timeout=300)
    if r.returncode != 0 and ("libasan" in r.stderr or "libubsan" in r.stderr):
        pytest.skip("sanitizer runtime libraries are not installed")
    assert r.returncode == 0, r.stderr[-4000:]


def _run(exe, cwd):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "abort_on_error=0:halt_on_error=1:detect_stack_use_after_return=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], cwd=cwd, capture_output=True, text=True, timeout=300, env=env)
    report = r.stdout[-2000:] + r.stderr[-6000:]
    assert r.returncode == 0, report
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, report
    return r.stdout


def test_host_abi_under_sanitizers(tmp_path):
    _need("g++")
    if not os.path.isdir(os.path.join(HIP_INCLUDE, "hip")):
        pytest.skip("HIP headers not installed")
    exe = str(tmp_path / "kvq_api_driver")
    _build(["g++", "-std=c++17", *SAN_FLAGS, "-Wall", "-Wextra", "-Wno-unused-parameter",
            f"-I{HIP_INCLUDE}", "-D__HIP_PLATFORM_AMD__", f"-I{CSRC}",
            os.path.join(SAN, "kvq_api_driver.cpp"), os.path.join(CSRC, "kvq_api.cpp"), "-o", exe],
           str(tmp_path))
    out = _run(exe, str(tmp_path))
    assert "kvq_api_driver ok" in out


def test_oracle_under_sanitizers(tmp_path):
    _need("gcc")
    exe = str(tmp_path / "oracle_driver")
    # the oracle's own arithmetic flags: every fp32 operation a single IEEE operation
    _build(["gcc", "-std=c11", *SAN_FLAGS, "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
            "-Wno-unknown-pragmas", os.path.join(SAN, "oracle_driver.c"),
            os.path.join(ROOT, "oracle", "kvq_oracle.c"), "-o", exe, "-lm"],
           str(tmp_path))
    out = _run(exe, str(tmp_path))
    assert "oracle_driver ok" in out
