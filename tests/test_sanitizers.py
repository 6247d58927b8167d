"""The CPU oracle and the C ABI's host code under the host sanitizers (AddressSanitizer and
UndefinedBehaviorSanitizer), no GPU.

oracle/oracle.c is rebuilt with gcc -fsanitize=address,undefined and every oracle pin
(tests/test_oracle.py) runs against that build; capi.cpp (argument validation, the workspace
arithmetic, the scratch lookup of the no-allocation entry point) is rebuilt with the sanitizers on
its host code only (-Xarch_host) and linked with the library's other objects, and the C-ABI host
checks (tests/test_capi_host.py) run against it.  Each runs in a child process that preloads the
compiler's sanitizer runtime; any report aborts it.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1", "OMP_NUM_THREADS": "2"}


def _run_child(test_file, env_extra, preload):
    env = dict(os.environ, **SAN_ENV, **env_extra, LD_PRELOAD=preload)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", test_file)], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
    return r.stdout


def test_oracle_pins_under_asan_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    lib = tmp_path / "liboracle_san.so"
    subprocess.run([gcc, "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wall", "-Wextra",
                    os.path.join(ROOT, "oracle", "oracle.c"), "-o", str(lib), "-lm"], check=True)
    rt = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    out = _run_child("test_oracle.py", {"LCA_ORACLE_LIB": str(lib)}, rt)
    assert " passed" in out


def test_capi_host_checks_under_asan_ubsan(tmp_path):
    hipcc = shutil.which("hipcc")
    rts = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if hipcc is None or not rts:
        pytest.skip("no hipcc / clang ASan runtime")
    from long_context_attention_22_amd import build as B
    csrc = os.path.join(ROOT, "long_context_attention_22_amd", "csrc")
    objs = []
    for src in B.SOURCES:
        obj = str(tmp_path / (src + ".o"))
        san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host",
               "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"] if src == "capi.cpp" else []
        subprocess.run([hipcc, *B.FLAGS, *B.EXTRA.get(src, []), *san, "-x", "hip", "-c", os.path.join(csrc, src),
                        "-o", obj], check=True, capture_output=True)
        objs.append(obj)
    lib = str(tmp_path / "liblca_san.so")
    subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                    "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", "-o", lib, *objs], check=True,
                   capture_output=True)
    out = _run_child("test_capi_host.py", {"LCA_LIB": lib}, rts[0])
    assert " passed" in out
