"""Build libtq.so (HIP, gfx950) in-tree with hipcc.

    python -m quantized_kv_cache_tq_amd.build [-j N] [-v]

Objects go to quantized_kv_cache_tq_amd/lib/obj, the library to
quantized_kv_cache_tq_amd/lib/libtq.so, and the benchmark's floor kernels
(tq_floor.hip) to quantized_kv_cache_tq_amd/lib/libtq_floor.so.  Every call recompiles every source.
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(PKG, "csrc")
LIB_DIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIB_DIR, "libtq.so")
SOURCES = ["tq_api.hip", "tq_set_rows.hip", "tq_decode.hip", "tq_decode_fused4.hip", "tq_prefill.hip",
           "tq_int8.hip"]
# benchmark floors (empty launch, one streaming read): not part of libtq
FLOOR_SOURCE = "tq_floor.hip"
FLOOR_LIB = os.path.join(LIB_DIR, "libtq_floor.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-FP32 instructions (v_pk_{add,mul,fma}_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-fast-math", "-ffp-contract=off", "-fno-gpu-rdc",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
]
# Per-source additions: the compiler's instruction-level-parallelism
# scheduling strategy, for the kernels it measured faster on (the prefill and
# int8 kernels, and the fused decode kernel's one-block variants, which have
# a translation unit of their own for this: the other decode kernels measured
# slower with it, set_rows too).
_MAX_ILP = ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]
SOURCE_FLAGS = {"tq_decode_fused4.hip": _MAX_ILP, "tq_prefill.hip": _MAX_ILP, "tq_int8.hip": _MAX_ILP}


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; a ROCm toolchain is required to build libtq")
    return path


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(LIB_DIR, "obj", os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(SRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, flush=True)
    return obj


def build(jobs: int = 4, verbose: bool = False) -> str:
    os.makedirs(os.path.join(LIB_DIR, "obj"), exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    # the benchmark's launch and streaming floors: a library of their own
    fobj = _compile(FLOOR_SOURCE, verbose)
    tmp = FLOOR_LIB + ".tmp"
    r = subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", fobj, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, FLOOR_LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=4)
    ap.add_argument("-v", action="store_true")
    a = ap.parse_args()
    print(build(a.j, a.v))
