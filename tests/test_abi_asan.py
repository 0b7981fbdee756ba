"""The C ABI's host-side validation under AddressSanitizer (CPU only).

Builds a host-only copy of the library (every csrc/*.hip compiled with
--offload-host-only and an empty device binary: no device code, so no kernel
can be launched; the HIP runtime loads code objects only when a kernel is
first launched, so the empty binary is never read) with
AddressSanitizer on the host side, links the C driver tests/asan/abi_host_check.c
against it, and runs it: sizes for valid configurations, documented statuses
and messages for invalid arguments, and no memory error that ASan can see in
the host code (config checks, scratch layout, argument validation, error
formatting).  The GPU build is untouched.
"""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decoder_block_rmsnorm_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "asan", "abi_host_check.c")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                                reason="ROCm toolchain not installed")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ... failed:\n{err}\n{r.stdout}"
    return r


def test_abi_host_validation_under_asan(tmp_path):
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    empty = tmp_path / "empty.fatbin"
    empty.write_bytes(b"")
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "--offload-host-only",
             "-Xclang", "-fcuda-include-gpubinary", "-Xclang", str(empty),
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC, *flags, "-c", src, "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(compile_one, srcs))
    lib = str(tmp_path / "libllama_block_asan.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address", "-o", lib, *objs,
          "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lrocprofiler-sdk-roctx"])
    exe = str(tmp_path / "abi_host_check")
    # (the driver is plain C, built by the host compiler: ASan's runtime comes with the executable)
    _run([CLANG, "-O1", "-g", "-fsanitize=address", "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
          DRIVER, "-o", exe, lib, f"-Wl,-rpath,{tmp_path}", "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, f"rc {r.returncode}\n{r.stdout}\n{r.stderr[-4000:]}"
    assert "ERROR: AddressSanitizer" not in r.stderr
    line = [l for l in r.stdout.splitlines() if l.startswith("ABI host checks:")]
    assert line, r.stdout
    n_ok, n_all = line[0].split(":")[1].split(" of ")
    assert int(n_ok) == int(n_all.split()[0]) > 100
