"""Build libqmm.so (the C-ABI library) for gfx950 with hipcc, in-tree, and
libqmm_ceiling.so (the benchmark's measurement kernels: plain streaming read and
register-only MFMA loop).

    python -m gemm_affine_u4_amd.build        # or __graft_entry__.build()
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libqmm.so")
CEILING_OUT = os.path.join(PKG, "libqmm_ceiling.so")
BUILD_DIR = os.path.join(ROOT, "_build")

# (source, extra flags, object): the GEMV and GEMM sources are built once per code width.
WIDTHS = (2, 3, 4, 6, 8)
SOURCES = ([("qmm_api.cpp", [], "qmm_api.o"), ("qmm_validate.cpp", [], "qmm_validate.o"),
            ("moe_route.hip", [], "moe_route.o"), ("bmv_u4.hip", [], "bmv_u4.o"),
            ("qmm_noalloc.hip", [], "qmm_noalloc.o"), ("gemv_step.hip", [], "gemv_step.o"),
            ("moe_gemm.hip", [], "moe_gemm.o")]
           + [(src, [f"-DQMM_BITS={b}"], f"{src.split('.')[0]}_b{b}.o") for src in ("gemv_u4.hip", "gemm_u4.hip")
              for b in WIDTHS]
           + [(src, ["-DQMM_BITS=8", "-DQMM_FP8=1"], f"{src.split('.')[0]}_f8.o")
              for src in ("gemv_u4.hip", "gemm_u4.hip")])

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
# Packed fp32 ops are kept out of the device code (compiler-generated v_pk_*_f32).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC, "-Wall"]


def _compile(entry) -> str:
    src, extra, obj_name = entry
    obj = os.path.join(BUILD_DIR, obj_name)
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stderr or "").splitlines() if noise not in ln and ln.strip()]
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


CEILING = ("ceiling.hip", [], "ceiling.o")


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(jobs: int = 8) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES + [CEILING]))
    _link(objs[:-1], OUT)
    _link(objs[-1:], CEILING_OUT)
    return OUT


if __name__ == "__main__":
    print(build())
