"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU
only, no device is touched).

Two builds, each in its own process with its own sanitizer runtime preloaded
into Python:

- the CPU oracle, built by g++ with -fsanitize=address,undefined; the CPU
  tests of the oracle and of the parity rules then run on it;
- the HIP library with its host code sanitized (clang's runtime: the device
  code is built as usual); the C-ABI tests, which exercise every host-side
  check of descriptions and tensors, then run on it.

A planted heap overflow and a planted signed overflow, each in a small
library built the same way, must be reported in the same setting, so that a
clean run is not a sanitizer that never loaded.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SRC = os.path.join(ROOT, "oracle", "mla_oracle.cpp")
LIB_SRCS = [os.path.join(ROOT, "head_latent_attention_amd", "csrc", f) for f in ("mla_prolog.hip", "mla_sfa.hip")]
HIPCC = os.environ.get("HIPCC", "hipcc")

CANARY = r"""
#include <cstdlib>
#include <climits>
extern "C" int heap_overflow(int i) { int* p = static_cast<int*>(std::malloc(4 * sizeof(int)));
  p[0] = 1; int v = p[i]; std::free(p); return v; }
extern "C" int signed_overflow(int a) { return a + INT_MAX; }
"""


def gcc_runtime(name):
    path = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def clang_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def run_python(code_or_args, env):
    full = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
                **env)
    args = code_or_args if isinstance(code_or_args, list) else ["-c", code_or_args]
    return subprocess.run([sys.executable, *args], cwd=ROOT, env=full, capture_output=True, text=True)


def canary_reports(lib, env):
    """The planted heap overflow and signed overflow are both reported."""
    # the heap overflow is reported by ASan, or first by UBSan's object-size
    # check of the same load
    for call, what in (("heap_overflow(4)", ("heap-buffer-overflow", "insufficient space")),
                       ("signed_overflow(5)", ("signed integer overflow",))):
        r = run_python(f"import ctypes; L = ctypes.CDLL({lib!r}); L.{call}", env)
        assert r.returncode != 0 and any(w in r.stderr for w in what), (call, r.returncode, r.stderr[-2000:])


@pytest.fixture(scope="module")
def work(tmp_path_factory):
    return tmp_path_factory.mktemp("sanitizers")


def test_oracle_under_asan_ubsan(work):
    asan, ubsan = gcc_runtime("libasan.so"), gcc_runtime("libubsan.so")
    if not (shutil.which("g++") and asan and ubsan):
        pytest.skip("g++ or its sanitizer runtimes are not installed")
    flags = ["-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer", "-shared", "-fPIC", "-pthread"]
    canary_src = work / "canary.cpp"
    canary_src.write_text(CANARY)
    canary = str(work / "libcanary_gcc.so")
    subprocess.run(["g++", *flags, str(canary_src), "-o", canary], check=True)
    lib = str(work / "libmla_oracle_san.so")
    subprocess.run(["g++", *flags, "-ffp-contract=off", "-fno-fast-math", ORACLE_SRC, "-o", lib], check=True)
    env = {"LD_PRELOAD": f"{asan}:{ubsan}", "MLA_ORACLE_LIBRARY": lib}
    canary_reports(canary, env)
    r = run_python(["-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                    "tests/test_oracle.py", "tests/test_oracle_sfa.py", "tests/test_parity_rules.py"], env)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-3000:]


def test_library_host_code_under_asan_ubsan(work):
    rt = clang_runtime()
    if not (shutil.which(HIPCC) and rt):
        pytest.skip("hipcc or clang's sanitizer runtime is not installed")
    clangxx = os.path.join(os.path.dirname(os.path.dirname(os.path.dirname(os.path.dirname(
        os.path.dirname(os.path.dirname(rt)))))), "bin", "clang++")
    host = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-shared-libasan"]
    canary_src = work / "canary.cpp"
    canary_src.write_text(CANARY)
    canary = str(work / "libcanary_clang.so")
    subprocess.run([clangxx, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-shared-libasan", "-shared", "-fPIC", str(canary_src), "-o", canary], check=True)
    lib = str(work / "libmla_prolog_san.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-mllvm", "-amdgpu-mfma-vgpr-form=1", *host, "-o", lib, *LIB_SRCS], check=True)
    env = {"LD_PRELOAD": rt, "MLA_PROLOG_LIBRARY": lib}
    canary_reports(canary, env)
    r = run_python(["-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider", "tests/test_abi.py"], env)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-3000:]
