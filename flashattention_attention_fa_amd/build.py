"""Build libfa_amd.so (the C ABI of include/fa.h) from csrc/ with hipcc for
gfx950, and libfa_ceiling.so (include/fa_ceiling.h: the measurement kernels
the benchmark's --ceilings mode runs).  Objects go to _build/ at the
repository root; the shared libraries are written next to this file, where
the Python binding and the benchmark load them."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
LIB = PKG / "libfa_amd.so"
CEILING_LIB = PKG / "libfa_ceiling.so"
CEILING_SOURCES = ["fa_ceiling.hip"]
BUILD_DIR = ROOT / "_build"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_fwd_fp8.hip", "fa_bwd.hip", "fa_decode.hip"]
# Per-source extra flags.  The forward kernel keeps its MFMA accumulators in
# vector registers (the softmax reads S directly, O stays put); without this
# the compiler parks them in accumulation registers and copies them back and
# forth every iteration.
SOURCE_FLAGS = {"fa_fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "fa_fwd_fp8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
# Packed fp32 VALU instructions are switched off for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-I", str(ROOT / "include"), "-I", str(CSRC)] + DEVICE_FLAGS


def _run(cmd, log):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "not a recognized feature" not in l)
    if log and out.strip():
        print(out, file=sys.stderr)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, resource_report: bool = False) -> Path:
    """Compile every source and link the library.  Always recompiles."""
    BUILD_DIR.mkdir(exist_ok=True)
    extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_report else []

    def compile_one(name):
        obj = BUILD_DIR / (name + ".o")
        _run([HIPCC, *COMMON, *SOURCE_FLAGS.get(name, []), *extra, "-c", str(CSRC / name),
              "-o", str(obj)],
             verbose or resource_report)
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES) + len(CEILING_SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES + CEILING_SOURCES))
    for lib, names in ((LIB, SOURCES), (CEILING_LIB, CEILING_SOURCES)):
        tmp = lib.with_name(f"{lib.name}.tmp{os.getpid():x}")
        _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", str(tmp),
              *(str(o) for o, n in zip(objs, SOURCES + CEILING_SOURCES) if n in names),
              "-Wl,-rpath,/opt/rocm/lib"], verbose)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, resource_report="--report" in sys.argv))
