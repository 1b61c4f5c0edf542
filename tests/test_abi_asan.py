"""The C ABI's host code under AddressSanitizer (CPU only).

Builds the library a second time with the host side of every source
instrumented (`-Xarch_host -fsanitize=address`; device code is untouched),
then runs the ABI tests of test_abi.py against that build in a child Python
with the sanitizer runtime preloaded.  Every argument check, workspace query
and status string then runs under ASan: an out-of-bounds read or a
use-after-free in the validation code fails the run."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_diffusion_draft_ctx_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "asan")
ROCM = "/opt/rocm"
SOURCES = ["api.cpp", "verify.hip", "attention.hip", "gemm.hip", "tree.hip", "draft.hip"]


def _asan_runtime():
    r = subprocess.run([os.path.join(ROCM, "llvm", "bin", "clang"),
                        "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isfile(path) else None


def _build():
    import concurrent.futures as cf
    os.makedirs(OUT, exist_ok=True)
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
             "-I", os.path.join(ROOT, "include")]

    def one(src):
        obj = os.path.join(OUT, src + ".o")
        r = subprocess.run([os.path.join(ROCM, "bin", "hipcc"), *flags, "-x", "hip", "-c",
                            os.path.join(CSRC, src), "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(one, SOURCES))
    lib = os.path.join(OUT, "libdflash_asan.so")
    r = subprocess.run([os.path.join(ROCM, "llvm", "bin", "clang++"), "-shared",
                        "-fsanitize=address", "-shared-libsan", *objs,
                        "-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
                        "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", lib],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return lib


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="the ABI tests with fake pointers run on CPU hosts")
def test_abi_checks_under_address_sanitizer():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime in this toolchain")
    lib = _build()
    env = dict(os.environ, DFLASH_LIBRARY=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in r.stderr, tail
    assert " passed" in r.stdout, tail
