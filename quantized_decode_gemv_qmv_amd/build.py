"""Builds libqmv.so (the HIP kernels and the C ABI of include/qmv.h) for gfx950.

Every HIP source is compiled with hipcc into an object under _build/, in
parallel, and linked into a shared library next to this file.  Packed FP32
instructions are disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libqmv.so")
# (source, object, extra flags): the dense vector and matrix-core kernels are
# compiled once per weight format so that those instantiations build in
# parallel
FORMATS = {0: "q8_0", 1: "q4_k", 2: "iq4_xs", 3: "q5_k", 4: "q6_k", 5: "q8g128"}
# the formats with a matrix-core decode, whose kernels are compiled per format too
MX_FORMATS = (0, 1, 2, 5)
SOURCES = ([(s, os.path.splitext(s)[0], []) for s in
            ("qmv_api.hip", "qmv_variants.hip", "qmv_quant.hip", "qmv_moe.hip", "qmv_router.hip",
             "qmv_measure.hip")]
           + [("qmv_matvec.hip", f"qmv_matvec_{n}", [f"-DQMV_MATVEC_FMT={f}"]) for f, n in FORMATS.items()]
           + [("qmv_mfma.hip", f"qmv_mfma_{FORMATS[f]}", [f"-DQMV_MX_FMT={f}"]) for f in MX_FORMATS]
           + [("qmv_mxf.hip", f"qmv_mxf_{FORMATS[f]}", [f"-DQMV_MX_FMT={f}"]) for f in MX_FORMATS])
ARCH = os.environ.get("QMV_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
            "-mcode-object-version=5", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(entry, extra: list[str]) -> str:
    src, name, defs = entry
    obj = os.path.join(BUILD, name + ".o")
    cmd = [hipcc(), *flags(), *defs, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 target feature
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if msg.strip():
        print(msg)
    return obj


def build(extra: list[str] | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    extra = list(extra or [])
    with cf.ThreadPoolExecutor(max_workers=min(os.cpu_count() or 8, 16, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
