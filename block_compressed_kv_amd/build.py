"""Build liblbca.so (hand-written HIP for gfx950) in-tree.

    python -m block_compressed_kv_amd.build          # compile every source, link
    python -m block_compressed_kv_amd.build --check  # also print the exported symbols

Each translation unit is compiled separately (in parallel) with hipcc for
gfx950 only, then linked into ``block_compressed_kv_amd/liblbca.so`` next to
the binding that loads it.  Packed-fp32 instruction selection is disabled on the
device pass (``-packed-fp32-ops``).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblbca.so")
SOURCES = ["api.cpp", "pool.hip", "pool_grad.hip", "cache.hip", "decode.hip", "decode_wide.hip", "attend_f32.hip", "prefill.hip", "index.hip", "gemm.hip", "attn_grad.hip"]
# measured-ceiling probes for the benchmark report (a library of their own, not the attention path)
CEIL_LIB = os.path.join(PKG, "libceilings.so")
CEIL_SOURCES = ["ceilings.hip"]
ARCH = "gfx950"


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build liblbca)")


def flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC, "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
    ]


def _compile(src):
    obj = os.path.join(BUILD, src + ".o")
    cmd = [_hipcc(), *flags(), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{' '.join(cmd)}\n{err}")
    return obj, err


def _link(objs, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + CEIL_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 4)) as ex:
        results = dict(zip(srcs, ex.map(_compile, srcs)))
    for obj, err in results.values():
        if err.strip() and verbose:
            print(err, file=sys.stderr)
    _link([results[s][0] for s in SOURCES], LIB, verbose)
    _link([results[s][0] for s in CEIL_SOURCES], CEIL_LIB, verbose)
    return LIB


if __name__ == "__main__":
    build()
    if "--check" in sys.argv:
        out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
        print("\n".join(l for l in out.splitlines() if " T " in l and ("lbca" in l or "csa" in l)))
