"""Build libmgemm.so in-tree with hipcc for gfx950.

Every translation unit under ``csrc/`` is compiled in parallel, then linked
into ``dense_gemm_12_amd/libmgemm.so``.  Run ``python -m dense_gemm_12_amd.build``
(``--changed``: recompile only sources older than their object files'
dependencies).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmgemm.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

# -packed-fp32-ops: never emit packed fp32 VALU ops (v_pk_{add,mul,fma}_f32).
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(os.path.dirname(HERE), "include"),
]


# Per-source flags: keep MFMA accumulators in VGPRs.  In the AGPR form the
# register allocator gives the last MFMA of each accumulator chain a fresh
# AGPR tuple and rotates all of them back at the loop edge (hundreds of
# v_accvgpr moves per K slice).  Every fp32 tile, and every 16-bit tile but
# the 256 x 256 ones of four waves (256 accumulators per lane, which need
# AGPRs and whose loops are clean), fits in VGPRs at its occupancy, so the
# flag is per file.
_VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
FILE_FLAGS = {"kernels_f32.hip": _VGPR_FORM, "kernels_f16_vgpr.hip": _VGPR_FORM,
              "kernels_bf16_vgpr.hip": _VGPR_FORM}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _stale(src: str, obj: str) -> bool:
    """An object is rebuilt when it is older than its source, any header
    under csrc/, the public header or this script."""
    if not os.path.exists(obj):
        return True
    deps = [src, __file__, os.path.join(os.path.dirname(HERE), "include", "mgemm.h")]
    deps += [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hpp")]
    t = os.path.getmtime(obj)
    return any(os.path.getmtime(d) > t for d in deps)


def _compile(src: str, extra: list[str], force: bool = True) -> str:
    obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
    if not force and not extra and not _stale(src, obj):
        return obj
    cmd = [HIPCC, *COMMON, *FILE_FLAGS.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(jobs: int | None = None, extra: list[str] | None = None, verbose: bool = False,
          force: bool = True) -> str:
    """Compile every source (with force=False only the stale ones) and link
    the shared library; returns its path."""
    os.makedirs(OUT_DIR, exist_ok=True)
    extra = list(extra or [])
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, force), srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True, force="--changed" not in sys.argv)
