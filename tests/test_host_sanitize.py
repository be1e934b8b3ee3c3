"""The library's host code under AddressSanitizer, LeakSanitizer and
UndefinedBehaviorSanitizer (CPU only).

tests/host_c/host_sanitize.cpp is linked with the library's sources, built
with the sanitizers on the host side only (each -fsanitize= behind
-Xarch_host: the device code is built as in the product library, and GPU
sanitizers are not part of this test).  The program walks the ring
arithmetic, the split schedule of an attention call, the attention
workspace layout, arena sizing on random configurations, the threaded RoPE
fill and the argument validation of every entry point; a sanitizer report
or a failed check fails the test.  No call reaches a GPU.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "kv_cache_attention_rtv_amd", "csrc")
BUILD = os.path.join(ROOT, "_build", "tests", "sanitize")
CLANG = "/opt/rocm/llvm/bin/clang++"

SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
FLAGS = ["-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument", *SANITIZE,
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]
SOURCES = [os.path.join(CSRC, s) for s in ("rtv_host.cpp", "append.hip", "attend.hip", "gemm.hip")] + \
          [os.path.join(HERE, "host_c", "host_sanitize.cpp")]


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    res = subprocess.run([CLANG, *FLAGS, "-c", src, "-o", obj], capture_output=True, text=True)
    return obj, res


@pytest.mark.skipif(not os.path.exists(CLANG) or shutil.which("ld") is None,
                    reason="the ROCm clang toolchain is not installed")
def test_host_code_is_clean_under_sanitizers():
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as pool:
        built = list(pool.map(_compile, SOURCES))
    for obj, res in built:
        assert res.returncode == 0, res.stdout + res.stderr
    exe = os.path.join(BUILD, "host_sanitize")
    res = subprocess.run([CLANG, "--hip-link", *SANITIZE, *[o for o, _ in built], "-o", exe,
                          "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "runtime error" not in run.stderr and "Sanitizer" not in run.stderr, run.stderr
    got = dict(line.rsplit(" ", 1) for line in run.stdout.strip().splitlines())
    for group in ("ring", "schedule", "workspace", "sizing", "rope", "validation"):
        assert got[f"{group} failures"] == "0", run.stdout + run.stderr
    assert int(got["ring_windows"]) > 100000
    # (creation up to its first device call runs only where there is no device)
    assert got.get("create_without_device", "1") == "1"
