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


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer build of the same
# sources (argument checks, plan builder, launch code): every sanitizer flag
# applies to the host compilation only, the gfx950 code is built as usual.
# Loaded into a Python process it needs the sanitizer runtime preloaded
# (see hostsan_runtime()).
HOSTSAN_LIB_PATH = os.path.join(HERE, "libmla_decode_hostsan.so")
HOSTSAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                 "-Xarch_host", "-shared-libsan"]


def hostsan_runtime() -> str:
    """Path of the clang AddressSanitizer runtime matching hipcc's host compiler."""
    r = subprocess.run([HIPCC.replace("hipcc", "amdclang++") if HIPCC.endswith("hipcc") else HIPCC,
                        "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        import glob
        cands = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        if not cands:
            raise RuntimeError("clang AddressSanitizer runtime not found")
        path = cands[0]
    return path


def build(verbose: bool = False, extra_flags=(), hostsan: bool = False, out_path: str = "") -> str:
    """Compile and link; returns the library path. ``hostsan`` builds the
    host-sanitized variant (beside the library unless ``out_path`` is given)
    instead of the library."""
    srcs = sources()
    out_path = out_path or (HOSTSAN_LIB_PATH if hostsan else LIB_PATH)
    flags = list(extra_flags) + (HOSTSAN_FLAGS if hostsan else [])
    with tempfile.TemporaryDirectory(prefix="mla_build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(s) + ".o") for s in srcs]
        jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
        with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
            warns = list(ex.map(lambda so: _compile(so[0], so[1], flags), zip(srcs, objs)))
        if verbose:
            for s, w in zip(srcs, warns):
                if w.strip():
                    print(f"--- {os.path.basename(s)}\n{w}", file=sys.stderr)
        tmp_lib = out_path + ".tmp"
        cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp_lib, *objs]
        if hostsan:
            cmd += HOSTSAN_FLAGS
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        os.replace(tmp_lib, out_path)
    return out_path


# Test-only probe library (tests/tile_probe): the decode kernels' building
# blocks run one at a time, for the tile tests.
PROBE_SRC = os.path.join(os.path.dirname(HERE), "tests", "tile_probe", "tile_probe.hip")
PROBE_LIB_PATH = os.path.join(os.path.dirname(PROBE_SRC), "libtile_probe.so")


def build_probe() -> str:
    tmp_lib = PROBE_LIB_PATH + ".tmp"
    cmd = [HIPCC, "-x", "hip", "-shared", "-fPIC", PROBE_SRC, "-o", tmp_lib, *COMMON_FLAGS]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for the tile probe:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp_lib, PROBE_LIB_PATH)
    return PROBE_LIB_PATH


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv, hostsan="--hostsan" in sys.argv)
    print(path)
