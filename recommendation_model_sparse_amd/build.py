"""Build the HIP library ``libdlrm_sparse.so`` for gfx950 (in-tree, with hipcc).

``python -m recommendation_model_sparse_amd.build`` compiles every source under
``csrc/`` to an object in ``_build/`` and links the shared library next to this
file.  Each call rebuilds everything.
"""
from __future__ import annotations

import os
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdlrm_sparse.so")
ARCH = os.environ.get("DLRM_OFFLOAD_ARCH", "gfx950")

# packed fp32 VALU forms are kept out of the generated code
HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas"]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def build(verbose: bool = False, extra_flags=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    t0 = time.time()
    procs = []
    objs = []
    for src in sources():
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc, *HIPCC_FLAGS, *extra_flags, *lang, "-c", src, "-o", obj]
        procs.append((src, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, cmd, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the device-only target feature; that note is harmless
        lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l or "error" in l]
        if p.returncode != 0:
            failed.append(src)
            sys.stderr.write(f"[build] FAILED {src}\n" + "\n".join(lines) + "\n")
        elif verbose and lines:
            sys.stderr.write("\n".join(lines) + "\n")
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB + f".tmp{os.getpid()}"
    # hipBLASLt runs the plain GEMMs of the dense layers (mlp.hip)
    subprocess.check_call([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs, "-lhipblaslt"])
    os.replace(tmp, LIB)
    if verbose:
        sys.stderr.write(f"[build] {LIB} in {time.time() - t0:.1f}s\n")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
