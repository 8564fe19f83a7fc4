"""Build libqsparse.so (HIP, gfx950) in-tree with hipcc.

    python -m top_kv_block_amd.build

Objects go to _build/ at the repository root; the shared library is written next to
this file, where the Python binding loads it.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqsparse.so")
SOURCES = ["metadata.hip", "select.hip", "probe.hip", "attn.hip", "fused.hip", "importance.hip", "qsparse_abi.hip"]
ARCH = os.environ.get("QSPARSE_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed-FP32 VALU ops (v_pk_fma_f32 and friends) in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _hipcc():
    for p in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if p and os.path.exists(p):
            return p
    return "hipcc"


def _compile(src):
    obj = os.path.join(OBJ, src.replace(".hip", ".o"))
    cmd = [_hipcc(), *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    return obj, errs


def build(verbose: bool = True) -> str:
    """Compile every HIP source and link the shared library. Always rebuilds."""
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        results = list(ex.map(_compile, SOURCES))
    for (obj, errs), src in zip(results, SOURCES):
        if errs.strip() and verbose:
            print(f"[{src}] {errs}", file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *[r[0] for r in results]]
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
