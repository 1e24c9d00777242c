"""The host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

api.cpp (argument validation, plan and workspace layout, dispatch) is compiled again with host-only
sanitizers and linked with the already built kernel objects; the ABI tests then run against that
library in a child process with the sanitizer runtime preloaded. Every call there stops at its
host-side validation, so no GPU is needed. Skipped when the kernel objects have not been built yet
(python -m fp4_compressed_sparse_kv_amd.build) or the toolchain has no sanitizer runtime.
"""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "fp4_compressed_sparse_kv_amd")
OBJ = os.path.join(PKG, "_build")
KERNEL_OBJS = ["quant", "index", "select", "poolsel", "attn", "prefill", "noalloc", "project"]


def _runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.mark.timeout(600)
def test_abi_validation_clean_under_host_sanitizers(tmp_path):
    hipcc = "/opt/rocm/bin/hipcc"
    rt = _runtime()
    objs = [os.path.join(OBJ, f"{n}.o") for n in KERNEL_OBJS]
    if not os.path.exists(hipcc) or rt is None:
        pytest.skip("no hipcc or no clang sanitizer runtime")
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("kernel objects not built")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer"]
    api_o = str(tmp_path / "api_san.o")
    lib = str(tmp_path / "libcsa2_san.so")
    subprocess.run([hipcc, "-x", "hip", "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
                    f"-I{os.path.join(ROOT, 'include')}", f"-I{os.path.join(PKG, 'csrc')}", *san,
                    "-c", os.path.join(PKG, "csrc", "api.cpp"), "-o", api_o],
                   check=True, capture_output=True, text=True)
    subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *san, "-shared-libsan", api_o, *objs,
                    "-o", lib], check=True, capture_output=True, text=True)
    child = (
        "import sys, pytest\n"
        "import fp4_compressed_sparse_kv_amd as C\n"
        f"C.LIB_PATH = {lib!r}\n"
        "assert C.lib()._name == C.LIB_PATH\n"
        "sys.exit(pytest.main(['-q', '-m', 'not gpu', '-p', 'no:cacheprovider', 'tests/test_abi.py']))\n"
    )
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-c", child], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=500)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
