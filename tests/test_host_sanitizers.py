"""AddressSanitizer and UndefinedBehaviorSanitizer over the library's host code.

The library is rebuilt from the current sources with both sanitizers on its
host half only (its device code is compiled as usual and never runs here), and
the host-only ABI tests (``test_abi.py``: sizes, layouts, every validation
path, stage timing, the binding's argument checks) run against that build in a
child process with the sanitizer runtime preloaded.  Any sanitizer report, or a
failing test, fails this test.
"""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "hierarchical_sparse_attention_mean_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "host_sanitizers")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/llvm/bin/clang++"

# every sanitizer flag applies to the host compilation only
HOST_SANITIZERS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                   "-Xarch_host", "-fno-omit-frame-pointer"]
COMPILE = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-w"]


def _runtime() -> str:
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return r.stdout.strip()


def _build() -> str:
    os.makedirs(OUT, exist_ok=True)

    def one(src):
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        r = subprocess.run([HIPCC, *COMPILE, *HOST_SANITIZERS, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        return obj

    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(one, srcs))
    lib = os.path.join(OUT, "liblighthouse_sanitized.so")
    rtdir = os.path.dirname(_runtime())
    r = subprocess.run([CLANGXX, "-shared", "-fPIC", "-shared-libsan", "-fsanitize=address,undefined", *objs,
                        "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", f"-Wl,-rpath,{rtdir}",
                        "-o", lib], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return lib


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="ROCm compilers not found")
def test_host_code_under_asan_and_ubsan():
    lib = _build()
    env = dict(os.environ)
    env.update(LH_LIBRARY=lib, LD_PRELOAD=_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # -s: reports written to stderr reach this process instead of pytest's capture
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-s", "-q",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0 and " passed" in out and "failed" not in out, out[-4000:]
