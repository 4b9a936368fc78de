"""Build libpkm.so (HIP for gfx950) in place: ``python -m product_key_memory_pkm_amd.build``.

Also builds libpkm_probe.so, the benchmark's peak probes (streaming read, MFMA loop), kept out of the library."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libpkm.so")
PROBE_OUT = os.path.join(PKG, "libpkm_probe.so")
BUILD = os.path.join(ROOT, "_build")

SOURCES = ["api.hip", "gather.hip", "score_topk.hip", "score_select.hip", "merge_softmax.hip", "merge_gather.hip",
           "gemm.hip", "bn.hip", "sort.hip", "value_grad.hip", "subkey_grad.hip", "diagnostics.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I" + os.path.join(ROOT, "include"),
         # packed fp32 VALU ops stay off (correctness of some packed forms is not trusted here)
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-result"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []

    def compile_one(src):
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        _run([HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose:
            print("compiled", src, flush=True)
        return obj

    with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, SOURCES + ["probe.hip"]))
    probe_obj = objs.pop()
    tmp = OUT + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, OUT)
    tmp = PROBE_OUT + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", probe_obj, "-o", tmp])
    os.replace(tmp, PROBE_OUT)
    if verbose:
        print("linked", OUT, "and", PROBE_OUT, flush=True)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
