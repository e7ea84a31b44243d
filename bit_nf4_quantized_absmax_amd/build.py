"""Builds libqlora_mi355x.so in-tree with hipcc for gfx950.

    python -m bit_nf4_quantized_absmax_amd.build        (or build() from Python)

Every .hip file under csrc/ is compiled to an object in _build/ (in
parallel) and linked into bit_nf4_quantized_absmax_amd/libqlora_mi355x.so.
Flags that matter for results:
  -ffp-contract=off            the codec's fp32 product-then-sum steps must
                               not fuse into FMAs (bit-exact decode)
  -packed-fp32-ops disabled    no v_pk_{add,mul,fma}_f32 in any kernel
IEEE fp32 division (hipcc's default) is kept; never build with -ffast-math.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB_NAME = "libqlora_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = os.environ.get("QLORA_OFFLOAD_ARCH", "gfx950")

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libqlora_mi355x")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src, extra):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc()] + COMMON_FLAGS + extra + ["-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), res.stderr))
    # host-side warnings about the gfx-only target feature are expected
    return obj


def build(verbose=False, extra_flags=()):
    """Compile every kernel source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    extra = list(extra_flags)
    workers = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), res.stderr))
    os.replace(tmp, LIB_PATH)
    if verbose:
        print("built", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
