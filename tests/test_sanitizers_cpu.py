"""CPU sanitizer run: the C ABI's host logic (kda_api.cpp: argument
validation, workspace carving, kernel selection) and the C oracle, each built
with g++/gcc under AddressSanitizer and UndefinedBehaviorSanitizer, driven by
the CPU ABI tests and the oracle pins in a child process that preloads the
sanitizer runtimes. Kernel launches are stubbed (tests/sanitize/host_stubs.cpp);
the GPU code is not built here. Any sanitizer report fails the child (halt on
the first error), and so this test."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_92_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                                reason="needs gcc and g++")


def _runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_host_abi_and_oracle_under_asan_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("sanitizer runtimes not installed")
    host_lib = str(tmp_path / "libkda_hostcheck.so")
    oracle_lib = str(tmp_path / "libkda_oracle_san.so")
    # __align__ and HIP_SYMBOL come from the HIP compiler's device headers, which g++
    # does not see
    subprocess.run(["g++", "-std=c++17", "-shared", "-fPIC", "-D__HIP_PLATFORM_AMD__",
                    "-D__align__(x)=__attribute__((aligned(x)))", "-DHIP_SYMBOL(x)=x",
                    "-I/opt/rocm/include", f"-I{ROOT}/include", f"-I{CSRC}"] + SAN +
                   [os.path.join(CSRC, "kda_api.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "host_stubs.cpp"), "-o", host_lib],
                   check=True)
    subprocess.run(["gcc", "-std=gnu99", "-shared", "-fPIC"] + SAN +
                   [os.path.join(ROOT, "oracle", "kda_oracle.c"), "-o", oracle_lib, "-lm",
                    "-lpthread"], check=True)
    env = dict(os.environ)
    env.update({"LD_PRELOAD": f"{asan}:{ubsan}",
                "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
                "KDA_HOST_CHECK_LIB": host_lib, "KDA_ORACLE_LIB": oracle_lib})
    # the child loads the sanitized builds, not the in-tree libraries
    probe = ("import ctypes, os\n"
             "from gated_delta_rule_92_amd import _lib\n"
             "import oracle.oracle as o\n"
             "assert _lib.LIB_PATH == os.environ['KDA_HOST_CHECK_LIB']\n"
             "assert _lib.load().kda_host_check_build() == 1\n"
             "assert o._load()._name == os.environ['KDA_ORACLE_LIB']\n")
    res = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-2000:]
    # and the sanitizer setup catches a planted heap overflow
    bad_src = tmp_path / "overflow.c"
    bad_src.write_text("#include <stdlib.h>\nint overflow(void) { int* p = malloc(4 * sizeof(int));"
                       " p[4] = 1; int r = p[0]; free(p); return r; }\n")
    bad_lib = str(tmp_path / "liboverflow.so")
    subprocess.run(["gcc", "-shared", "-fPIC"] + SAN + [str(bad_src), "-o", bad_lib], check=True)
    res = subprocess.run([sys.executable, "-c",
                          f"import ctypes; ctypes.CDLL({bad_lib!r}).overflow()"],
                         env=env, capture_output=True, text=True, timeout=300)
    assert res.returncode != 0 and ("heap-buffer-overflow" in res.stderr or
                                   "runtime error:" in res.stderr)
    tests = [os.path.join(ROOT, "tests", f) for f in
             ("test_abi_cpu.py", "test_oracle_pins.py", "test_oracle_backward.py",
              "test_oracle_epilogue.py")]
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                          "-p", "no:cacheprovider"] + tests,
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (res.stdout[-3000:] + res.stderr[-3000:])
    print(tail)
    assert res.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail
