"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two builds, each exercised by the existing host tests in a child process with
the sanitizer runtime preloaded; any report aborts the child and fails the
test:
 - the oracle (oracle/mhc_oracle.cpp), built with clang and
   -fsanitize=address,undefined, runs its pins (tests/test_oracle_pins.py,
   tests/test_stack_conditioning.py);
 - libmhc with its host code sanitized (every csrc source through hipcc,
   the sanitizer flags on the host pass only; the device code is the usual
   gfx950 build), runs the C-ABI host checks (tests/test_capi_host.py):
   argument validation, size queries, status strings, aliasing rules.
No GPU is needed: nothing here launches a kernel.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang++"
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CSRC = os.path.join(ROOT, "mhc_hyper_connections_amd", "csrc")
SOURCES = ["capi.cpp", "pre.hip", "pre8.hip", "pre_fused.hip", "post.hip", "amax.hip", "bwd.hip", "noalloc.hip"]
SAN = ["-fsanitize=address", "-fsanitize=undefined"]


def _runtime():
    out = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _child_env(**extra):
    env = dict(os.environ)
    env.update(extra)
    env["LD_PRELOAD"] = _runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


def _run_tests(files, env):
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider", *files]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    text = res.stdout + res.stderr
    assert res.returncode == 0, text[-4000:]
    for marker in ("AddressSanitizer", "runtime error:", "UndefinedBehaviorSanitizer"):
        assert marker not in text, text[-4000:]
    return text


needs_toolchain = pytest.mark.skipif(not (os.path.exists(CLANG) and os.path.exists(HIPCC)),
                                     reason="ROCm clang / hipcc not available")


@needs_toolchain
def test_oracle_under_asan_and_ubsan(tmp_path):
    if _runtime() is None:
        pytest.skip("no ASan runtime")
    lib = tmp_path / "libmhc_oracle_san.so"
    subprocess.run([CLANG, "-O1", "-g", "-std=c++17", "-fPIC", "-shared", "-fno-omit-frame-pointer",
                    "-fno-fast-math", *SAN, "-fno-sanitize-recover=all", "-shared-libasan",
                    "-o", str(lib), os.path.join(ROOT, "oracle", "mhc_oracle.cpp")], check=True)
    out = _run_tests(["tests/test_oracle_pins.py", "tests/test_stack_conditioning.py"],
                     _child_env(MHC_TEST_ORACLE_LIB=str(lib)))
    assert " passed" in out


@needs_toolchain
def test_capi_host_code_under_asan_and_ubsan(tmp_path):
    if _runtime() is None:
        pytest.skip("no ASan runtime")

    def compile_one(src):
        obj = tmp_path / (os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17",
               "-fno-omit-frame-pointer", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-sanitize-recover=all", "-c", os.path.join(CSRC, src), "-o", str(obj)]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-3000:]
        return str(obj)

    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    lib = tmp_path / "libmhc_san.so"
    subprocess.run([CLANG, "-shared", "-fPIC", *SAN, "-shared-libasan", "-o", str(lib), *objs,
                    "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], check=True)
    out = _run_tests(["tests/test_capi_host.py"], _child_env(MHC_TEST_LIBMHC=str(lib)))
    assert " passed" in out
