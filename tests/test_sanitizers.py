"""Host sanitizer builds (CPU): the fp64 oracle, the pair store and the C ABI's
host code, each built with AddressSanitizer and UndefinedBehaviorSanitizer
(no recovery) and driven by a small program under tests/sanitize/.  The ABI
build is a host-only pass of api.cpp linked with stand-ins for the kernel
launchers, so it exercises argument validation, workspace sizes, status
strings and the launch-failure path without device code."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, (" ".join(cmd) + "\n" + r.stdout[-3000:] + r.stderr[-3000:])
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", *SAN_FLAGS, "-fsanitize=address,undefined", "-o", exe, os.path.join(SAN, "oracle_main.c"),
          os.path.join(ROOT, "oracle", "hypic_oracle.c"), "-lm"])
    assert "ok" in _run([exe], env=ENV)


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_store_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "store_san")
    _run(["g++", "-std=c++17", *SAN_FLAGS, "-fsanitize=address,undefined", "-o", exe,
          os.path.join(SAN, "store_main.cpp"), os.path.join(ROOT, "state_caching_segment_amd", "csrc", "store.cpp")])
    assert "ok" in _run([exe], env=ENV)


@pytest.mark.skipif(not os.path.exists(CLANG) or not os.path.exists("/opt/rocm/lib/libamdhip64.so"),
                    reason="ROCm clang or HIP runtime not available")
def test_api_host_code_under_asan_ubsan(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include")]
    host = ["-std=c++17", *SAN_FLAGS, "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    objs = []
    for src, hip in ((os.path.join(ROOT, "state_caching_segment_amd", "csrc", "api.cpp"), True),
                     (os.path.join(SAN, "launch_stubs.hip"), True),
                     (os.path.join(SAN, "api_main.cpp"), False)):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        lang = ["-x", "hip", "--cuda-host-only", "--offload-arch=gfx950"] if hip else []
        _run([CLANG, *lang, *host, *inc, "-c", src, "-o", obj])
        objs.append(obj)
    exe = str(tmp_path / "api_san")
    _run([CLANG, "-fsanitize=address,undefined", "-o", exe, *objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib"])
    assert "ok" in _run([exe], env=ENV)
