"""Builds libattn119.so (HIP C++ for gfx950) in-tree with hipcc.

    python -m exact_attention_119_amd.build [-j JOBS] [-v]

Every source is compiled to an object under exact_attention_119_amd/_build/ in
parallel, then linked into exact_attention_119_amd/libattn119.so.  Always
rebuilds: the call is the "does it compile" check.
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libattn119.so")
ARCH = "gfx950"

SOURCES = [
    "api.cpp",
    "blockmap.hip",
    "fwd_bf16_d128.hip",
    "fwd_bf16_d64.hip",
    "fwd_fp8p_d128.hip",
    "fwd_fp8p_d64.hip",
    "fwd_fp8qk8_d128.hip",
    "fwd_fp8qk8_d64.hip",
    "fwd_fp8pv_d128.hip",
    "fwd_count_d128.hip",
    "fwd_count_d64.hip",
    "quant.hip",
    "bwd.hip",
]

# -packed-fp32-ops: hipcc must not emit v_pk_{add,mul,fma}_f32 (the host pass warns
# that it does not know the feature; that warning is harmless).
# -mno-amdgpu-ieee -fno-honor-nans: the kernels never produce or consume NaN on their
# arithmetic path (masked scores are -inf, which these flags keep); without them
# every fmaxf of an MFMA result is preceded by a quieting v_max_f32.  The one NaN the
# kernels write (a poisoned batch row) is a stored bit pattern.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
          "-fno-honor-nans"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libattn119.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "is not a recognized feature" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(jobs: int = 8, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else ["-x", "hip"]
        cmds.append([cc, *COMMON, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([cc, "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", "--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args(argv)
    print(build(args.jobs, args.verbose))


if __name__ == "__main__":
    sys.exit(main())
