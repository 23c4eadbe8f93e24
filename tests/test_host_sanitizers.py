"""libca2's host code under AddressSanitizer + UndefinedBehaviorSanitizer
(CPU only). The host source is compiled as plain C++ with the sanitizers,
linked with the kernel objects of the regular build (device code is not
instrumented), and tests/host_sanitizer_driver.cpp drives every pure host
function and every validation path through the C ABI. Any sanitizer report,
leak or failed check fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "causal_kv_cache_amd")
BUILD = os.path.join(PKG, "_build")
CLANG = "/opt/rocm/llvm/bin/clang++"
KERNEL_OBJS = ["temporal_attn.o", "spatial_attn.o", "cache_write.o", "qkv_proj.o", "toy_block.o"]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def _have_toolchain():
    return os.path.exists(CLANG) and all(os.path.exists(os.path.join(BUILD, o)) for o in KERNEL_OBJS)


@pytest.mark.skipif(not _have_toolchain(), reason="needs ROCm clang++ and the built kernel objects")
def test_host_code_under_asan_ubsan(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"), "-I", "/opt/rocm/include",
           "-D__HIP_PLATFORM_AMD__"]
    host_o, drv_o, exe = (str(tmp_path / n) for n in ("host.o", "driver.o", "driver"))
    common = [CLANG, "-std=c++17", "-O1", "-g"] + SAN + inc
    for src, obj in ((os.path.join(PKG, "csrc", "ca2_host.cpp"), host_o),
                     (os.path.join(ROOT, "tests", "host_sanitizer_driver.cpp"), drv_o)):
        r = subprocess.run(common + ["-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
    objs = [os.path.join(BUILD, o) for o in KERNEL_OBJS]
    r = subprocess.run([CLANG] + SAN + [drv_o, host_o] + objs +
                       ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    supp = tmp_path / "lsan.supp"
    # allocations the HIP / HSA runtimes make at initialisation and keep for the process
    supp.write_text("leak:libamdhip64\nleak:libhsa-runtime64\nleak:librocprofiler\nleak:libdrm\n")
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:exitcode=23"
    env["LSAN_OPTIONS"] = f"suppressions={supp}"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "host checks passed" in out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
