"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

The library is relinked with ``csrc/mlp_api.hip`` (every argument check, the tile and schedule
planners, the workspace layout, the host-only calls) compiled with host-side sanitizers; the other
objects are the normal build's. ``tests/abi_check/abi_check.c``, built with the same sanitizers,
then calls every entry point with arguments its validation must reject (so nothing reaches a
GPU) and the host-only calls over a grid of valid, edge and invalid descriptors. A memory error or
undefined behaviour aborts the program; a wrong status makes it exit non-zero."""
import glob
import os
import subprocess

import pytest

from gated_mlp_gemms_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
# host-side only: each -fsanitize= of a hipcc line follows -Xarch_host (device code stays as built)
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def _objects_current() -> bool:
    objs = glob.glob(os.path.join(B.BUILD, "*.o"))
    if not objs or not os.path.exists(B.LIB):
        return False
    built = min(os.path.getmtime(o) for o in objs)
    srcs = glob.glob(os.path.join(B.CSRC, "*")) + glob.glob(os.path.join(ROOT, "include", "*.h"))
    return all(os.path.getmtime(s) <= built for s in srcs)


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


def test_host_code_under_asan_and_ubsan(tmp_path):
    if not (os.path.exists(B.HIPCC) and os.path.exists(CLANG)):
        pytest.skip("the ROCm compilers are not installed")
    if not _objects_current():
        B.build()
    san_obj = str(tmp_path / "mlp_api_san.o")
    _run([B.HIPCC, *B.CFLAGS, *HOST_SAN, "-c", os.path.join(B.CSRC, "mlp_api.hip"), "-o", san_obj])
    objs = [o for o in glob.glob(os.path.join(B.BUILD, "*.o")) if os.path.basename(o) != "mlp_api.o"]
    lib = str(tmp_path / "libgated_mlp_san.so")
    _run([B.HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-o", lib, *objs, san_obj])
    exe = str(tmp_path / "abi_check")
    _run([CLANG, "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g",
          "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "abi_check", "abi_check.c"), "-o", exe,
          lib, f"-Wl,-rpath,{tmp_path}", "-Wl,-rpath,/opt/rocm/lib", "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "all checks passed" in r.stdout
