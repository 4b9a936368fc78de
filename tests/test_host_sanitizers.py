"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The C ABI's host side (argument checks, workspace layout, handle life cycle,
error strings) is compiled a second time with the sanitizers on the host pass
only (`-Xarch_host` before each flag; device code is untouched), linked with
the regular objects of the other sources, and the ABI tests of test_abi.py are
run against that copy in a child process with the ASan runtime preloaded.
None of those tests launches a kernel, so no GPU is needed.  A sanitizer report
fails the child (halt_on_error), and so this test.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT_DIR = os.path.join(ROOT, "_build", "hostsan")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def _build_sanitized():
    """Every source compiled afresh into its own folder (never the in-tree library's objects, which
    may predate the sources): api.hip with the host sanitizers, the others as the regular build does."""
    from concurrent.futures import ThreadPoolExecutor

    from product_key_memory_pkm_amd import build as B
    os.makedirs(OUT_DIR, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]

    def compile_one(src):
        obj = os.path.join(OUT_DIR, src.replace(".hip", ".o"))
        if src == "api.hip":
            flags = [f for f in B.FLAGS if f != "-O3"] + ["-O1", "-g"] + san
        else:
            flags = list(B.FLAGS)
        B._run([HIPCC, *flags, "-c", os.path.join(B.CSRC, src), "-o", obj])
        return obj

    with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, B.SOURCES))
    lib = os.path.join(OUT_DIR, "libpkm.so")
    B._run([HIPCC, "-shared", "-fPIC", f"--offload-arch={B.ARCH}", *san, *objs, "-o", lib])
    return lib


@pytest.mark.timeout(600)
def test_abi_checks_under_address_and_ub_sanitizers():
    rt = _asan_runtime()
    if rt is None or not os.path.exists(HIPCC):
        pytest.skip("hipcc or the clang ASan runtime is not installed")
    lib = _build_sanitized()
    env = dict(os.environ)
    env.update(PKM_LIB_PATH=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=24")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
                        "-m", "not gpu", "-p", "no:cacheprovider", "-p", "no:xdist"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=540)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout, out[-2000:]
