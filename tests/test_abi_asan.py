"""The host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is rebuilt with the sanitizers on its host code only (device code is compiled as
usual) into a temporary directory, and the host ABI tests (argument validation, buffer checks,
KV-share binding rules, workspace sizes, status strings: no device work) run against it in a
child process with the sanitizer runtime preloaded.  Any out-of-bounds access, use after free
or undefined behaviour in those paths ends the child with a report.
"""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from hybrid_attention_ssm_swa_amd import build as B   # noqa: E402

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def _build(out):
    def comp(src):
        obj = os.path.join(out, src + ".o")
        r = subprocess.run([B._hipcc(), *B.COMMON, *SAN, "-c", os.path.join(B.CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        return obj
    with cf.ThreadPoolExecutor(min(8, len(B.SOURCES))) as ex:
        objs = list(ex.map(comp, B.SOURCES))
    lib = os.path.join(out, "libhymba_mixer.so")
    r = subprocess.run([B._hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *SAN, "-shared-libsan", "-o", lib,
                        *objs, "-L/opt/rocm/lib", "-lhipblaslt", "-Wl,-rpath,/opt/rocm/lib"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return lib


def test_host_abi_under_asan_and_ubsan():
    rt = _runtime()
    if rt is None:
        pytest.skip("no clang AddressSanitizer runtime in this ROCm install")
    try:
        B._hipcc()
    except RuntimeError:
        pytest.skip("hipcc not found")
    with tempfile.TemporaryDirectory() as out:
        lib = _build(out)
        syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
        assert "__asan_report" in syms and "__ubsan_handle" in syms, "the host code is not instrumented"
        code = ("import sys; sys.path.insert(0, 'tests')\n"
                "import hybrid_attention_ssm_swa_amd._lib as L\n"
                f"L.load_library({lib!r})\n"
                "assert L.load_library()._name == " + repr(lib) + "\n"
                "import pytest\n"
                "sys.exit(pytest.main(['tests/test_abi_host.py', '-q', '-p', 'no:cacheprovider']))\n")
        env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
        r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                           timeout=600)
        tail = (r.stdout + r.stderr)[-4000:]
        assert r.returncode == 0, tail
        assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
