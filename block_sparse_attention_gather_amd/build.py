"""Build libbsa.so (HIP for gfx950) in-tree.

    python -m block_sparse_attention_gather_amd.build [--jobs N] [--verbose] [--no-trace]

Each .hip translation unit is compiled to an object in parallel (the two attention sources
with a machine-scheduling strategy of their own, SOURCE_FLAGS), then linked into
block_sparse_attention_gather_amd/libbsa.so.  The same sources with -DBSA_TRACE (per-workgroup
timestamps of the attention launch, read back with bsa_trace_read) are linked into
libbsa_trace.so, a debug library for load-balance measurements.  Always recompiles (a build
check must compile).
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
LIB = os.path.join(PKG, "libbsa.so")
TRACE_LIB = os.path.join(PKG, "libbsa_trace.so")
SOURCES = ["api.hip", "reorder.hip", "route.hip", "attn.hip", "attn_fp8.hip", "fp8.hip"]
ARCH = os.environ.get("BSA_OFFLOAD_ARCH", "gfx950")

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-fvisibility=hidden",
    "-I", os.path.join(ROOT, "include"),
    # packed fp32 ops (v_pk_*_f32) are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]

# Per-source compiler options: LLVM machine-scheduling strategies that order each attention
# loop faster than the default on the Wan-480p layer (same arithmetic in another instruction
# order, bitwise-identical outputs).  attn.hip: "max-ilp", 1.2 % faster (max-memory-clause and
# the iterative strategies slower or equal).  attn_fp8.hip: "iterative-ilp", 1.3 % faster with
# the ExpCast cast and 0.9 % with the exact one (max-ilp, max-memory-clause and
# iterative-minreg slower or equal).
SOURCE_FLAGS = {"attn.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
                "attn_fp8.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libbsa)")


_FEATURE_PROBE = """#include <hip/hip_runtime.h>
__global__ void bsa_feature_probe(float* x) { x[threadIdx.x] *= 2.0f; }
"""


def check_device_flags(cc: str) -> None:
    """Compile a one-line kernel for the device only with CFLAGS: the host pass of a full
    compile always warns that it does not know the packed-fp32 feature (harmless, and filtered
    from the build log below), but the device pass must accept it, or the flag that keeps
    packed fp32 instructions out of the code would silently do nothing."""
    os.makedirs(BUILD, exist_ok=True)
    src = os.path.join(BUILD, "feature_probe.hip")
    with open(src, "w") as fh:
        fh.write(_FEATURE_PROBE)
    cmd = [cc, *CFLAGS, "--offload-device-only", "-c", src,
           "-o", os.path.join(BUILD, "feature_probe.o")]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0 or "not a recognized feature" in r.stdout:
        raise RuntimeError("the device compiler does not accept the build's target features:\n"
                           + r.stdout)


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass of every compile warns about the device-only feature (check_device_flags
    # proves that the device pass accepts it)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}")
    if verbose and out.strip():
        print(out)


def _link(cc, objs, lib, verbose):
    tmp = lib + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp], verbose)
    os.replace(tmp, lib)


def build(jobs: int = 0, verbose: bool = False, trace: bool = True) -> str:
    cc = hipcc()
    os.makedirs(BUILD, exist_ok=True)
    check_device_flags(cc)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc, *CFLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src),
                     "-o", obj])
    trace_obj = os.path.join(BUILD, "attn_trace.o")
    if trace:
        cmds.append([cc, *CFLAGS, *SOURCE_FLAGS.get("attn.hip", []), "-DBSA_TRACE", "-c",
                     os.path.join(CSRC, "attn.hip"), "-o", trace_obj])
    with ThreadPoolExecutor(jobs or min(len(cmds), os.cpu_count() or 1)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    _link(cc, objs, LIB, verbose)
    if trace:
        _link(cc, [o for o in objs if not o.endswith("attn.o")] + [trace_obj], TRACE_LIB,
              verbose)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=0)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--no-trace", action="store_true", help="skip libbsa_trace.so")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose, trace=not a.no_trace))


if __name__ == "__main__":
    main(sys.argv[1:])
