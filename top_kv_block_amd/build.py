"""Build libqsparse.so and libqsparse_checked.so (HIP, gfx950) in-tree with hipcc.

    python -m top_kv_block_amd.build

Objects go to _build/ at the repository root; the shared libraries are written next to
this file, where the Python binding loads them. The checked library has the same kernels;
only its C ABI layer is compiled with QS_CHECKED (each call first checks the device-resident
tables it will use, and waits for that check).
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
LIB_CHECKED = os.path.join(PKG, "libqsparse_checked.so")
SOURCES = ["metadata.hip", "select.hip", "probe.hip", "attn.hip", "fused.hip", "importance.hip", "check.hip",
           "qsparse_abi.hip"]
ABI = "qsparse_abi.hip"
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


def _compile(job):
    src, checked = job
    obj = os.path.join(OBJ, src.replace(".hip", "_checked.o" if checked else ".o"))
    cmd = [_hipcc(), *HIPCC_FLAGS, *(["-DQS_CHECKED"] if checked else []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    return obj, errs


def _link(lib, objs):
    tmp = lib + ".tmp"
    subprocess.check_call([_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    """Compile every HIP source and link both shared libraries. Always rebuilds."""
    os.makedirs(OBJ, exist_ok=True)
    jobs = [(src, False) for src in SOURCES] + [(ABI, True)]
    with cf.ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        results = list(ex.map(_compile, jobs))
    for (obj, errs), (src, checked) in zip(results, jobs):
        if errs.strip() and verbose:
            print(f"[{src}{' checked' if checked else ''}] {errs}", file=sys.stderr)
    objs = {job: r[0] for job, r in zip(jobs, results)}
    _link(LIB, [objs[(src, False)] for src in SOURCES])
    _link(LIB_CHECKED, [objs[(src, src == ABI)] for src in SOURCES])
    if verbose:
        print(f"built {LIB} and {LIB_CHECKED}")
    return LIB


if __name__ == "__main__":
    build()
