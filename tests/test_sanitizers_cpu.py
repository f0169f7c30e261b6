"""Host-side sanitizer runs (no GPU): the oracle under AddressSanitizer and
UndefinedBehaviorSanitizer, and the C ABI's host code (argument validation,
error reporting) built with host-only AddressSanitizer and driven by the
plain-C client. Device code is never instrumented."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-4000:], r.stderr[-4000:])
    return r


def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-Wall", "-Wextra", "-Werror",
          "-o", exe, os.path.join(ROOT, "oracle", "oracle.c"),
          os.path.join(ROOT, "tests", "oracle_sanitize_driver.c"), "-lm"])
    r = _run([exe], env=dict(os.environ, ASAN_OPTIONS="abort_on_error=1:detect_leaks=1"))
    assert "oracle driver ok" in r.stdout and "runtime error" not in r.stderr


def _asan_runtime_dir():
    r = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        r = subprocess.run([CLANG, "-print-runtime-dir"], capture_output=True, text=True)
        path = os.path.join(r.stdout.strip(), "libclang_rt.asan-x86_64.so")
    return os.path.dirname(path) if os.path.exists(path) else None


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="needs hipcc and clang")
def test_abi_host_code_under_asan(tmp_path):
    rt = _asan_runtime_dir()
    if rt is None:
        pytest.skip("no clang AddressSanitizer runtime")
    csrc = os.path.join(ROOT, "bit_adamw_optimizer_amd", "csrc")
    common = ["-std=c++17", "-fPIC", "--offload-arch=gfx950", "-ffp-contract=off", "-Xclang", "-target-feature",
              "-Xclang", "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include"), "-I" + csrc]
    objs = []
    for src in ("abi.hip", "kernels.hip"):
        obj = str(tmp_path / (src + ".o"))
        extra = ["-O1", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"] \
            if src == "abi.hip" else ["-O3"]
        _run([HIPCC] + common + extra + ["-c", os.path.join(csrc, src), "-o", obj])
        objs.append(obj)
    lib = str(tmp_path / "libmsamp.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
          "-shared-libasan", "-o", lib] + objs)
    exe = str(tmp_path / "c_abi_smoke")
    _run([CLANG, "-std=c11", "-O1", "-g", "-fsanitize=address", "-shared-libasan", "-fno-omit-frame-pointer",
          "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROOT, "include"),
          os.path.join(ROOT, "tests", "c_abi_smoke.c"), "-L" + str(tmp_path), "-lmsamp",
          "-Wl,-rpath," + str(tmp_path), "-Wl,-rpath," + rt, "-o", exe])
    # the HIP runtime keeps allocations until exit: leak reports are off
    r = _run([exe], env=dict(os.environ, ASAN_OPTIONS="abort_on_error=1:detect_leaks=0"))
    assert "c abi ok" in r.stdout
