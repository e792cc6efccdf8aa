"""Build libdspark.so (HIP, gfx950) in-tree.

    python -m semi_autoregressive_drafting_amd.build

Each .hip file under csrc/ is compiled to an object in _build/ (in parallel),
then linked into semi_autoregressive_drafting_amd/libdspark.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdspark.so")
PROBE_SRC = os.path.join(PKG, "csrc_probe")
PROBE_LIB = os.path.join(PKG, "libdspark_probe.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results land in VGPRs, so epilogues read them without v_accvgpr_read
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    f"-I{os.path.join(ROOT, 'include')}",
    f"-I{CSRC}",
]


def _hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found (ROCm is required to build libdspark.so)")
    return exe


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def probe_sources():
    return sorted(os.path.join(PROBE_SRC, f) for f in os.listdir(PROBE_SRC) if f.endswith(".hip"))


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [_hipcc(), *HIPCC_FLAGS, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{out}")
    if verbose and out.strip():
        print(out)
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, out)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every HIP source for gfx950 and link libdspark.so (the drafting
    path) and libdspark_probe.so (the benchmark's pure-read ceiling); returns
    the path of libdspark.so."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    probe_srcs = probe_sources()
    jobs = jobs or min(len(srcs) + len(probe_srcs), 8)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs + probe_srcs))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], PROBE_LIB)
    return LIB


HOSTSAN_LIB = os.path.join(BUILD, "libdspark_hostsan.so")
HOST_SANITIZERS = ["-fno-omit-frame-pointer", "-g",
                   "-Xarch_host", "-fsanitize=address",
                   "-Xarch_host", "-fsanitize=undefined",
                   "-Xarch_host", "-fno-sanitize-recover=undefined"]


def asan_runtime() -> str | None:
    """The ASan runtime of the ROCm clang that built the library (it also
    carries the UBSan handlers), or None."""
    import glob
    hits = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(_hipcc())), "llvm", "lib",
                                         "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


def build_host_sanitized() -> str:
    """libdspark.so with its host layer (dspark_api.hip: argument validation,
    workspace sizing, launch planning) compiled with AddressSanitizer and
    UndefinedBehaviorSanitizer; the kernels' objects are the normal build's
    (build() must have run).  Load it with the ASan runtime preloaded
    (asan_runtime()) and DSPARK_LIB pointing at it."""
    os.makedirs(os.path.join(BUILD, "hostsan"), exist_ok=True)
    src = os.path.join(CSRC, "dspark_api.hip")
    obj = os.path.join(BUILD, "hostsan", "dspark_api.o")
    flags = [f for f in HIPCC_FLAGS if f != "-O3"] + ["-O1"]
    res = subprocess.run([_hipcc(), *flags, *HOST_SANITIZERS, "-c", src, "-o", obj],
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed on dspark_api.hip (sanitized):\n" + res.stderr)
    others = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o") for s in sources()
              if os.path.basename(s) != "dspark_api.hip"]
    missing = [o for o in others if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"build() first: {missing[0]} is missing")
    _link(others + [obj], HOSTSAN_LIB)
    return HOSTSAN_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
