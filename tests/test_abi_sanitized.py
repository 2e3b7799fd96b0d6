"""The ABI layer (abi.cpp: validation, workspace sizing, dispatch) built on the
host with AddressSanitizer and UndefinedBehaviorSanitizer, linked with the
library's kernel objects, and the host-side ABI tests (tests/test_abi.py) run
against it in a child process with the sanitizer runtime preloaded. Any
sanitizer report fails the test. No GPU is touched: every call in those tests
returns from host validation.

Needs the objects of a normal build (``_build/*.o``, written by
``__graft_entry__.build()``) and ROCm's clang with its sanitizer runtimes;
skipped when either is missing.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang++"


def _asan_runtime():
    found = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return found[0] if found else None


def test_abi_under_asan_and_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from transformer_attention_rope_amd import build as b
    objs = [os.path.join(b.BUILD, os.path.splitext(s)[0] + ".o") for s in b.SOURCES if s.endswith(".hip")]
    rt = _asan_runtime()
    if not os.path.exists(CLANG) or rt is None:
        pytest.skip("ROCm clang or its sanitizer runtime is missing")
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("kernel objects missing: run __graft_entry__.build() first")
    san = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer"]
    abi_o = str(tmp_path / "abi.o")
    lib = str(tmp_path / "libnc_attn.so")
    subprocess.run([CLANG, "-x", "c++", "-std=c++17", "-O1", "-g", "-fPIC", *san, "-D__HIP_PLATFORM_AMD__",
                    "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-c",
                    os.path.join(b.CSRC, "abi.cpp"), "-o", abi_o], check=True, capture_output=True)
    subprocess.run([CLANG, "-shared", *san, "-shared-libsan", "-o", lib, abi_o, *objs, "-L/opt/rocm/lib",
                    "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], check=True, capture_output=True)
    logs = str(tmp_path / "san")
    env = dict(os.environ, LD_PRELOAD=rt, NC_ATTN_LIBRARY=lib,
               ASAN_OPTIONS=f"detect_leaks=0:log_path={logs}",
               UBSAN_OPTIONS=f"print_stacktrace=1:halt_on_error=1:log_path={logs}")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    reports = "".join(open(f).read() for f in glob.glob(logs + "*"))
    assert r.returncode == 0 and not reports, f"{r.stdout[-2000:]}\n{r.stderr[-2000:]}\n{reports[:4000]}"
    assert "passed" in r.stdout
