"""Build the gfx950 library ``libmxfp4_moe.so`` in this package directory.

    python -m mxfp4_block_scaled_amd.build [-v]

Every HIP source is compiled for gfx950 only with hipcc; the host C ABI
(csrc/api.cpp) is compiled by hipcc as plain host C++. Objects go to
``_build/`` at the repository root; the shared library lands next to this
file, which is where the binding loads it from.
"""

from __future__ import annotations

import concurrent.futures
import os
import re
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libmxfp4_moe.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

HIP_SOURCES = ["bucket.hip", "gemv.hip", "gemv_rows.hip", "gemv_one.hip", "gemm.hip", "combine.hip", "route.hip", "gemm_mx.hip", "gemm_regdec.hip", "stream.hip", "noalloc.hip"]
HOST_SOURCES = ["api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _common_flags():
    return ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]


def _device_flags():
    # packed fp32 VALU ops are switched off for all device code
    return [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _resource_problems(remarks: str) -> list:
    """Kernels that use scratch memory or spill registers, from the
    compiler's resource-usage remarks."""
    bad, name = [], None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        # SGPR spills land in VGPR lanes (no memory) unless scratch is used,
        # which the scratch size shows
        m = re.search(r"(ScratchSize \[bytes/lane\]|VGPRs Spill): (\d+)", line)
        if m and int(m.group(2)) != 0:
            bad.append(f"{name}: {m.group(1)} = {m.group(2)}")
    return bad


def _compile(src: str, verbose: bool) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-c", path, "-o", obj] + _common_flags()
    if src.endswith(".hip"):
        cmd += _device_flags() + ["-Rpass-analysis=kernel-resource-usage"]
    else:
        cmd += ["-x", "c++", "-D__HIP_PLATFORM_AMD__"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    text = r.stdout + r.stderr
    out = "\n".join(line for line in text.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line and "remark:" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{out}")
    # every kernel must keep its state in registers and LDS: scratch memory
    # (private arrays or VGPR spills) costs a slow memory round trip per access
    bad = _resource_problems(text)
    if bad:
        raise RuntimeError(f"{src}: kernels use scratch memory or spill:\n  " + "\n  ".join(bad))
    if verbose and out.strip():
        print(out, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    sources = HIP_SOURCES + HOST_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(sources), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), sources))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking {LIB_NAME} failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv[1:]))
