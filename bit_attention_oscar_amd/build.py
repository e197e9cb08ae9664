"""Build liboscar_kv.so (gfx950) in-tree with hipcc.

Every HIP source is compiled with:
  --offload-arch=gfx950            MI355X only
  -ffp-contract=off                no implicit fused multiply-add (the
                                   quantizer needs one rounding per op; the
                                   kernels use explicit fmaf where they fuse)
  -fhip-fp32-correctly-rounded-divide-sqrt   IEEE fp32 division
  -Xclang -target-feature -Xclang -packed-fp32-ops   no packed fp32 VALU ops
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "liboscar_kv.so")

SOURCES = ["append.hip", "decode.hip", "prefill.hip", "prefill_attn.hip", "scratch.hip", "oscar_kv.cpp"]
# per-source extra flags: the decode kernels carry -inf but never NaN (NaN
# inputs are outside the cache contract), so max/min need no NaN quieting
EXTRA = {"decode.hip": ["-fno-honor-nans"]}
COMMON_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build liboscar_kv.so")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "not a recognized feature" not in l
                    and "ignoring feature" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        out = _run([cc, *COMMON_FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and out.strip():
            print(out)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


SANITIZED_LIB = os.path.join(BUILD_DIR, "liboscar_kv_sanitized.so")


def build_sanitized() -> str:
    """The host library (oscar_kv.cpp) built with AddressSanitizer and
    UndefinedBehaviorSanitizer on its host code only (each -fsanitize= after
    -Xarch_host), linked with the kernels' objects of a normal build(): for
    running the C-ABI argument checks under the sanitizers on the CPU.  Load
    it with the sanitizer runtime preloaded (sanitizer_runtime())."""
    if not all(os.path.exists(os.path.join(BUILD_DIR, src + ".o")) for src in SOURCES):
        build()
    cc = hipcc()
    san = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined".split()
    obj = os.path.join(BUILD_DIR, "oscar_kv.cpp.sanitized.o")
    flags = [f for f in COMMON_FLAGS if f != "-O3"] + ["-O1", "-g", "-fno-omit-frame-pointer"]
    _run([cc, *flags, *san, "-c", os.path.join(CSRC, "oscar_kv.cpp"), "-o", obj])
    objs = [os.path.join(BUILD_DIR, src + ".o") for src in SOURCES if src != "oscar_kv.cpp"] + [obj]
    _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *san, *objs, "-o", SANITIZED_LIB])
    return SANITIZED_LIB


def sanitizer_runtime() -> str:
    """Path of the AddressSanitizer runtime of the HIP toolchain's clang."""
    import glob
    root = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    for pat in (os.path.join(root, "lib", "llvm", "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so"),
                "/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"):
        hits = sorted(glob.glob(pat))
        if hits:
            return hits[-1]
    raise RuntimeError("AddressSanitizer runtime not found")


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
