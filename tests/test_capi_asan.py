"""The C ABI's host code (argument validation, size queries, workspace
arithmetic, descriptor and member-array reads) built with AddressSanitizer
and UndefinedBehaviorSanitizer on the host side only, and exercised by a C
driver (tests/capi_validation.c) whose calls never reach the GPU.  Device
code is built as usual: the sanitizers are host-only here."""

import concurrent.futures
import os
import shutil
import subprocess

import pytest

from bit_nf4_quantized_absmax_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CLANG = "/opt/rocm/llvm/bin/clang"
HOST_SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-sanitize-recover=all"


def _have_toolchain():
    try:
        B.hipcc()
    except RuntimeError:
        return False
    return os.path.exists(CLANG)


@pytest.mark.skipif(not _have_toolchain(), reason="needs hipcc and ROCm clang")
def test_capi_validation_under_host_sanitizers(tmp_path):
    flags = [f for f in B.COMMON_FLAGS if f != "-O3"] + ["-O1", "-g"] + HOST_SAN.split()

    def compile_one(src):
        obj = os.path.join(str(tmp_path), os.path.basename(src) + ".o")
        res = subprocess.run([B.hipcc()] + flags + ["-c", src, "-o", obj], capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-4000:]
        return obj

    with concurrent.futures.ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, B.sources()))
    lib = os.path.join(str(tmp_path), "libqlora_san.so")
    res = subprocess.run([B.hipcc(), "-shared", "-fPIC", "--offload-arch=" + B.ARCH] + HOST_SAN.split() +
                         ["-o", lib] + objs, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    exe = os.path.join(str(tmp_path), "capi_validation")
    res = subprocess.run([CLANG, "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                          os.path.join(HERE, "capi_validation.c"), "-o", exe, lib,
                          "-Wl,-rpath," + str(tmp_path), "-Wl,-rpath,/opt/rocm/lib"],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env.pop("LD_PRELOAD", None)
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0 and "capi validation ok" in res.stdout, (res.stdout + res.stderr)[-6000:]
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr[-6000:]
