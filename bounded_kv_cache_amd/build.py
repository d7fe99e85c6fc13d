"""Build the HIP library ``libprefix_sliding.so`` in-tree for gfx950.

Every kernel source is compiled with hipcc (one object per source, in
parallel) and linked into one shared library next to this file.  Packed fp32
instructions are disabled for all device code (-packed-fp32-ops)."""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libprefix_sliding.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["api.hip", "append.hip", "decode.hip", "prefill.hip", "backward.hip", "heavy.hip", "reset_pe.hip", "probe.hip"]
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def common_flags() -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]


def _compile(src: str, verbose: bool, extra=(), build_dir: str = BUILD_DIR) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *common_flags(), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = (res.stdout + res.stderr)
    # the host pass does not know the device-only feature flag: harmless
    out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if verbose and out.strip():
        print(out, file=sys.stderr)
    return obj


def build(verbose: bool = False, out: str = LIB_PATH, defines=(), build_dir: str = BUILD_DIR) -> str:
    """Compile every source and link ``out``.  ``defines`` (e.g. "PS_DECODE_WAVES=8")
    override the kernels' compile-time launch-shape defaults."""
    os.makedirs(build_dir, exist_ok=True)
    extra = [f"-D{d}" for d in defines]
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, extra, build_dir), SOURCES))
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
