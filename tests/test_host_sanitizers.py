"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Every HIP source is compiled with the sanitizers on its host side only (the
device code is built as usual and never runs here), linked with the C program
`tests/abi_host_checks.c`, and run.  That program drives the size and plan
queries over shapes at and beyond the ABI's limits, and every validation
failure of every entry point, with fake device pointers that validation must
reject before anything is enqueued.  Any out-of-bounds access, leak, signed
overflow or division by zero in the host code aborts it.  No GPU is used."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kv_cache_attention_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")

# sanitizers on the host pass only: each flag goes to the host compiler
HOST_SANITIZE = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-sanitize-recover=undefined".split()
C_SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]

pytestmark = pytest.mark.skipif(
    not (os.path.exists(HIPCC) and os.path.exists(CLANG) and os.path.exists(CLANGXX)),
    reason="needs ROCm's hipcc and clang")


def _run(cmd, timeout):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       timeout=timeout)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}"
    return r.stdout


def test_host_code_under_asan_and_ubsan(tmp_path):
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    objs = []
    procs = []
    for f in srcs:
        obj = str(tmp_path / (f[:-4] + ".o"))
        objs.append(obj)
        cmd = [HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *HOST_SANITIZE,
               "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, f), "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                            text=True)))
    for cmd, p in procs:
        out, _ = p.communicate(timeout=600)
        assert p.returncode == 0, f"{' '.join(cmd)}\n{out[-4000:]}"
    drv = str(tmp_path / "abi_host_checks.o")
    _run([CLANG, "-O1", "-g", *C_SANITIZE, "-I", INCLUDE, "-c",
          os.path.join(ROOT, "tests", "abi_host_checks.c"), "-o", drv], 120)
    exe = str(tmp_path / "abi_host_checks")
    lib = os.path.join(ROCM, "lib")
    _run([CLANGXX, *C_SANITIZE, drv, *objs, "-L", lib, "-lamdhip64", f"-Wl,-rpath,{lib}",
          "-o", exe], 120)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True,
                       timeout=300, env=env)
    assert r.returncode == 0, f"rc {r.returncode}\n{r.stdout}\n{r.stderr[-6000:]}"
    assert "host ABI checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-6000:]
