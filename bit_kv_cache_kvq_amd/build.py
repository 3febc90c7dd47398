"""Build libkvq.so (HIP, gfx950) in place with hipcc.

    python -m bit_kv_cache_kvq_amd.build
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["kvq_api.cpp", "kvq_append.hip", "kvq_decode.hip", "kvq_decode_v2.hip", "kvq_decode_v3.hip",
           "kvq_probe.hip", "kvq_noalloc.hip"]
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops are disabled for all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]
# Per-source extra flags.  The decode kernel's tile-counter atomic is issued by one lane and
# its return is read a tile later; the compiler's atomic optimizer would rewrite it as a
# wave-wide atomic whose result is broadcast (and waited for) on the spot.
SOURCE_FLAGS: dict[str, list[str]] = {
    "kvq_decode.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"],
    "kvq_decode_v2.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"],
    "kvq_decode_v3.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"],
}
BUILD_DIR = os.path.join(HERE, "_build")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libkvq.so")


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = [os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o") for src in SOURCES]
    cmds = [[HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), *(extra or []), "-c", os.path.join(CSRC, src), "-o", obj]
            for src, obj in zip(SOURCES, objs)]
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
