"""Build libkvq.so in place: hipcc for gfx950, one object per source, compiled in parallel.

Flags: -O3, no fast-math (HIP's default correctly rounded fp32 division is kept), and packed
fp32 arithmetic disabled (-Xclang -target-feature -Xclang -packed-fp32-ops).  f16 denormals must
stay enabled (the default): the decode kernels feed code fields to the matrix cores as exact f16
subnormals, so no denormal-flushing option may be added here.

`--qk-valu` builds the same sources with -DKVQ_QK_VALU=1 into libkvq_qkvalu.so: single-query MHA
8-bit symmetric caches then take QK on the vector ALU (v_dot2_f32_f16) instead of the matrix
cores.  That library exists to compare the two; the binding loads it when KVQ_LIBRARY names it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkvq.so")
LIB_QK_VALU = os.path.join(HERE, "libkvq_qkvalu.so")
SOURCES = ["kvq_host.hip", "kvq_append.hip"] + [
    f"kvq_decode_b{bits}{scheme}.hip" for bits in (2, 4, 8) for scheme in "sa"] + [
    "kvq_decode_b16.hip", "kvq_decode_b8f.hip", "kvq_decode_dense.hip"] + [
    f"kvq_decode_mix_k{bits}{scheme}.hip" for bits in (2, 4, 8) for scheme in "sa"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src: str, build_dir: str = BUILD, defines: tuple = ()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *(f"-D{d}" for d in defines), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out.strip():
        sys.stderr.write(out + "\n")
    return obj


def build(verbose: bool = True, qk_valu: bool = False) -> str:
    build_dir, lib = (BUILD + "_qkvalu", LIB_QK_VALU) if qk_valu else (BUILD, LIB)
    defines = ("KVQ_QK_VALU=1",) if qk_valu else ()
    os.makedirs(build_dir, exist_ok=True)
    # one hipcc per core, the largest translation units (the mixed-format kernels) first; each
    # takes a few GB, so one process per source at once could exhaust a small host's memory
    order = sorted(SOURCES, key=lambda s: not s.startswith("kvq_decode_mix"))
    with cf.ThreadPoolExecutor(max_workers=max(1, min(len(SOURCES), os.cpu_count() or 8))) as ex:
        done = dict(zip(order, ex.map(lambda s: _compile(s, build_dir, defines), order)))
    objs = [done[s] for s in SOURCES]
    tmp = lib + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(qk_valu="--qk-valu" in sys.argv[1:])
