"""Builds libmla_decode.so (gfx950 only) in this directory with hipcc.

    python -m mla_paged_kv_02_amd.build

Every source under csrc/ is compiled as HIP for gfx950; objects build in
parallel and link into one shared library. The build always recompiles.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_NAME = "libmla_decode.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-mcode-object-version=5",
    # keep the compiler from forming packed FP32 ops (v_pk_* f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") or f.endswith(".cpp"))


def _compile(src: str, obj: str, extra):
    cmd = [HIPCC, "-x", "hip", "-c", src, "-o", obj, *COMMON_FLAGS, *extra]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {os.path.basename(src)}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r.stderr


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile and link; returns the library path."""
    srcs = sources()
    with tempfile.TemporaryDirectory(prefix="mla_build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(s) + ".o") for s in srcs]
        jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
        with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
            warns = list(ex.map(lambda so: _compile(so[0], so[1], list(extra_flags)), zip(srcs, objs)))
        if verbose:
            for s, w in zip(srcs, warns):
                if w.strip():
                    print(f"--- {os.path.basename(s)}\n{w}", file=sys.stderr)
        tmp_lib = LIB_PATH + ".tmp"
        cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp_lib, *objs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        os.replace(tmp_lib, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
