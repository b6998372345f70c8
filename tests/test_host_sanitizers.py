"""The C ABI's host-side argument validation under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).  A copy of libprism is built with the sanitizers
on its host code (hipcc -Xarch_host, so the GPU code is built as usual), and the C driver
tests/host/abi_validation.c, built with the same clang and sanitizer runtime, calls every
entry point with malformed sizes, flags, pointers and workspace sizes.  Every call must
return its error status before touching the GPU, with no sanitizer report."""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "content_adaptive_block_zone_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.timeout(900)
def test_host_validation_under_asan_and_ubsan(tmp_path):
    rt = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not os.path.exists(CLANG) or not rt:
        pytest.skip("ROCm clang or its sanitizer runtime not found")
    rpath = f"-Wl,-rpath,{os.path.dirname(rt[0])}"
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), *SAN]

    def cc(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([HIPCC, *flags, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with cf.ThreadPoolExecutor(8) as ex:
        objs = list(ex.map(cc, sorted(glob.glob(os.path.join(CSRC, "*.hip")))))
    lib = str(tmp_path / "libprism_san.so")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-fsanitize=address,undefined",
                        "-shared-libsan", rpath, *objs, "-o", lib], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = str(tmp_path / "abi_validation")
    r = subprocess.run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                        "-shared-libsan", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                        "-D__HIP_PLATFORM_AMD__", os.path.join(ROOT, "tests", "host", "abi_validation.c"), lib,
                        f"-Wl,-rpath,{tmp_path}", rpath, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout[-4000:])
    report = r.stderr
    assert "AddressSanitizer" not in report and "runtime error" not in report, report[-4000:]
    assert r.returncode == 0, (r.stdout[-2000:], report[-2000:])
    assert "0 unexpected statuses" in r.stdout
