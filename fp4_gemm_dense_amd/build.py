"""Build the gfx950 HIP library ``libdg.so`` in-tree with hipcc.

Every source under ``csrc/`` is compiled for gfx950 only; the shared library is
written next to this file so that it travels with the source tree.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdg.so")
SOURCES = ["api.cpp", "planner.cpp", "fp8_gemm.hip", "fp8_gemm_wide.hip", "ffn.hip", "noalloc.hip", "skinny.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
COMMON = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # keep the compiler from forming packed-fp32 VALU ops (device code only; the
    # host pass may warn that it does not know this feature)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(os.path.dirname(HERE), "include"),
]


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    return src, obj, r


def build(verbose=False, extra=()):
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = []
    for src, obj, r in results:
        msg = (r.stdout + r.stderr).strip()
        noise = [ln for ln in msg.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
        if verbose and noise:
            print(f"[{src}]\n" + "\n".join(noise), file=sys.stderr)
        objs.append(obj)
    tmp = LIB + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp, *extra],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
