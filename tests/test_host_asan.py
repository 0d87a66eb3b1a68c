"""The C ABI's host code under AddressSanitizer (host only: the device code is
not instrumented).  Rebuilds the entry-point layer with ASan into a temporary
directory, links it with the already compiled kernels, and runs the ABI tests
against that library in a child process with the ASan runtime preloaded.
Every call there fails validation before any HIP call, so no GPU is needed."""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "dynamic_sparse_attention_paged_amd")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
sys.path.insert(0, ROOT)
from dynamic_sparse_attention_paged_amd.build import SOURCES  # noqa: E402

KERNEL_OBJS = [os.path.splitext(f)[0] + ".o" for f in SOURCES if f != "dsa_api.cpp"]


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm*/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_abi_under_host_asan(tmp_path):
    objs = [os.path.join(PKG, "_build", o) for o in KERNEL_OBJS]
    rt = _asan_runtime()
    if not os.path.exists(HIPCC) or rt is None or not all(os.path.exists(o) for o in objs):
        pytest.skip("needs hipcc, the clang ASan runtime and a prior build (__graft_entry__.build())")
    api_o = str(tmp_path / "dsa_api_asan.o")
    lib = str(tmp_path / "libdsa_asan.so")
    cc = [HIPCC, "-O1", "-g", "-fPIC", "-std=c++17", "--offload-arch=gfx950",
          "-I", os.path.join(ROOT, "include"),
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
          "-x", "hip", "-c", os.path.join(PKG, "csrc", "dsa_api.cpp"), "-o", api_o]
    subprocess.run(cc, check=True, capture_output=True)
    link = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950",
            "-Xarch_host", "-fsanitize=address", "-o", lib]
    subprocess.run(link + objs + [api_o], check=True, capture_output=True)
    runner = (
        "import sys; sys.path.insert(0, %r)\n"
        "import dynamic_sparse_attention_paged_amd._lib as L\n"
        "L.LIB_PATH = %r\n"
        "import pytest\n"
        "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', %r]))\n"
    ) % (ROOT, lib, os.path.join(ROOT, "tests", "test_abi.py"))
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")
    p = subprocess.run([sys.executable, "-c", runner], env=env, capture_output=True, text=True,
                       timeout=300)
    assert p.returncode == 0 and "ERROR: AddressSanitizer" not in p.stderr, \
        p.stdout[-2000:] + p.stderr[-2000:]
