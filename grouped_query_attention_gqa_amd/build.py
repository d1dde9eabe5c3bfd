"""Build libgqa.so (HIP, gfx950) in-tree.

    python -m grouped_query_attention_gqa_amd.build

Every ``csrc/*.hip`` file is compiled to an object with hipcc for gfx950 and
the objects are linked into ``grouped_query_attention_gqa_amd/libgqa.so``.
Packed-fp32 instructions are disabled in device code on purpose: the
compiler must not form v_pk_{add,mul,fma}_f32 from scalar or float2 code.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgqa.so")
ARCH = os.environ.get("GQA_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libgqa.so)")


COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


# Per-file additions.  decode_mfma.hip: its 32- and 64-row kernels run one
# wave per SIMD, where the compiler would otherwise put the matrix
# accumulators in AGPRs and copy all of them into VGPRs on every tile (176
# v_accvgpr moves per 16-key tile at 64 rows); the VGPR form keeps them where
# the softmax and the final merge use them.
FILE_FLAGS = {
    "decode_mfma.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc()] + COMMON_FLAGS + FILE_FLAGS.get(os.path.basename(src), []) + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libgqa.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


PROBE_DIR = os.path.join(HERE, "probe")
PROBE_LIB = os.path.join(HERE, "libgqa_probe.so")


def build_probe(verbose: bool = False) -> str:
    """libgqa_probe.so: measurement aids the bench uses beside the library
    (the sustained matrix-core rate); never linked into libgqa.so."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(PROBE_DIR, "*.hip")))
    objs = [_compile(s) for s in srcs]
    tmp = PROBE_LIB + ".tmp"
    r = subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs,
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print(f"built {PROBE_LIB}")
    return PROBE_LIB


if __name__ == "__main__":
    build(verbose=True)
    build_probe(verbose=True)
