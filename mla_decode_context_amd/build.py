"""Compile libmla.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmla.so")
# (source, extra flags).  MFMA operands and results stay in ordinary VGPRs
# (-amdgpu-mfma-vgpr-form=1): every kernel's accumulators fit in them, and that
# form needs no copies through the accumulator registers.
_VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
SOURCES = [
    ("mla_api.hip", []),
    ("mla_decode.hip", _VGPR_FORM),
    ("mla_merge.hip", _VGPR_FORM),
    ("mla_decode_h128.hip", _VGPR_FORM),
    ("mla_calib.hip", _VGPR_FORM),
]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops stay off: hipcc emits ordinary fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


# The host pass does not know the packed-fp32 feature flag; that warning (and
# the count line after it) is expected and dropped.  Nothing else is filtered.
_NOISE = ("is not a recognized feature for this target", "generated when compiling")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if not any(n in l for n in _NOISE) and l.strip())
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Always recompile (one object per source, then link); returns the library path."""
    objs = []
    for src, extra in SOURCES:
        obj = os.path.join(PKG, "_build", src.replace(".hip", ".o"))
        os.makedirs(os.path.dirname(obj), exist_ok=True)
        _run([hipcc(), *HIPCC_FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c",
              os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"], verbose)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
