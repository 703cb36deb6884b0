"""Build libfa.so (gfx950) in-tree with hipcc.

    python -m io_aware_tiled_10_amd.build [-v]

Each source under csrc/ is compiled to an object in _build/ (in parallel), then
linked into io_aware_tiled_10_amd/libfa.so.  A second build of the same sources with
FA_DEBUG_SYNC (every counted wait a full wait, every barrier draining the wave's
loads first) is linked into libfa_debugsync.so: a race canary that the tests compare
bit for bit with the first.  The benchmark's measurement aid (fa_ceiling.hip, the
sustained matrix-core rate on register-resident operands) is linked on its own into
libfa_ceiling.so.  Always recompiles.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa.so")
LIB_DEBUG_SYNC = os.path.join(PKG, "libfa_debugsync.so")
LIB_CEILING = os.path.join(PKG, "libfa_ceiling.so")
CEILING_SOURCE = "fa_ceiling.hip"
ARCH = "gfx950"

SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_bwd.hip", "fa_decode.hip", "fa_quant.hip"]

# Per-source extra flags.  Every kernel is built with IEEE NaN semantics: a NaN score
# must fail the forward's block-sum test (which -fno-honor-nans folds into a plain
# "greater than"), so NaN inputs reach the outputs that depend on them.
EXTRA: dict = {}

# Packed fp32 VALU forms are kept out of the generated code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libfa.so")


def _compile(src: str, verbose: bool, variant: str = "") -> str:
    os.makedirs(os.path.join(BUILD, variant), exist_ok=True)
    obj = os.path.join(BUILD, variant, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"]
    defs = ["-DFA_DEBUG_SYNC"] if variant == "debugsync" else []
    cmd = [hipcc(), *lang, *COMMON, *DEVICE_FLAGS, *defs, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src),
           "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(line for line in (r.stderr or "").splitlines()
                    if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    return obj


def _link(objs, out: str, verbose: bool) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(s, v) for v in ("", "debugsync") for s in SOURCES] + [(CEILING_SOURCE, "")]
    with ThreadPoolExecutor(max_workers=min(len(jobs), 8)) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], verbose, j[1]), jobs))
    n = len(SOURCES)
    _link(objs[:n], LIB, verbose)
    _link(objs[n:2 * n], LIB_DEBUG_SYNC, verbose)
    _link(objs[2 * n:], LIB_CEILING, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
