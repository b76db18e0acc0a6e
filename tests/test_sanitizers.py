"""Host code under AddressSanitizer / UndefinedBehaviorSanitizer (CPU only).

* The fp64 oracle (oracle/ttt_oracle.c) is compiled with gcc -fsanitize=address,undefined
  into tests/native/oracle_driver.c, which calls every oracle entry point on a tiny batched
  model (ragged and all-ignored chunks, two SGD steps, gradients, generation).
* The library's host code (every csrc/*.hip source; the device code is compiled as usual and
  never runs) is built with clang's AddressSanitizer into tests/native/abi_driver.cpp, which
  checks the C-ABI contract that needs no GPU: argument and configuration errors, the
  allocator hook, error messages, every call on a NULL context, TTT_ENODEV without a device.

A sanitizer report (heap or stack overflow, use after free, leak, undefined behaviour) makes
the program exit non-zero and the test fail with the report.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"


def _run(cmd, env=None, timeout=300):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    return r.returncode, r.stdout + r.stderr


def _sanitizer_env():
    env = dict(os.environ)
    env.update(ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")
    return env


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    rc, out = _run(["gcc", "-std=gnu11", "-O1", "-g", "-fopenmp", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    os.path.join(NATIVE, "oracle_driver.c"), "-o", exe, "-lm"])
    assert rc == 0, out
    rc, out = _run([exe], env=_sanitizer_env())
    assert rc == 0 and "all checks passed" in out, out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="ROCm toolchain not found")
def test_host_library_under_asan(tmp_path):
    import torch
    if torch.cuda.is_available():
        pytest.skip("checks the path without a device; the GPU tests cover the rest")
    csrc = os.path.join(ROOT, "test_token_chunk_amd", "csrc")
    srcs = sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith(".hip"))

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        # the sanitizer instruments the host side only (device code is built unchanged)
        return obj, _run([HIPCC, "--offload-arch=gfx950", "-x", "hip", "-O1", "-std=c++17", "-fPIC",
                          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
                          "-I", os.path.join(ROOT, "include"), "-I", csrc, "-Wno-unused-result",
                          "-c", src, "-o", obj])

    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        built = list(ex.map(compile_one, srcs))
    for obj, (rc, out) in built:
        assert rc == 0, out
    exe = str(tmp_path / "abi_driver")
    rc, out = _run([CLANGXX, "-std=c++17", "-O1", "-g", "-fsanitize=address", "-fno-omit-frame-pointer",
                    "-I", os.path.join(ROOT, "include"), os.path.join(NATIVE, "abi_driver.cpp"),
                    *[obj for obj, _ in built], "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
                    "-o", exe])
    assert rc == 0, out
    rc, out = _run([exe], env=_sanitizer_env())
    assert rc == 0 and "all checks passed" in out, out
    assert "AddressSanitizer" not in out and "LeakSanitizer" not in out, out
