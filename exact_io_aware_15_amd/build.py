"""Build libfa.so (the HIP kernels + C ABI) in-tree for gfx950 with hipcc.

    python -m exact_io_aware_15_amd.build

Each source compiles to an object in parallel; the objects link into
exact_io_aware_15_amd/libfa.so.  Always rebuilds.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libfa.so")
# debug-sync build: the tiled kernels fence every HBM -> LDS copy and every LDS read
# stage (FA_DEBUG_SYNC=1); tests compare it bitwise with libfa.so
OUT_DEBUG_SYNC = os.path.join(PKG, "libfa_debugsync.so")
BUILD_DIR = os.path.join(PKG, "_build")

SOURCES = ["fa_api.cpp", "fa_prefill_bf16.hip", "fa_prefill_f32.hip", "fa_decode.hip", "fa_backward.hip"]
DEBUG_SYNC_SOURCES = ["fa_prefill_bf16.hip", "fa_backward.hip"]  # the rest is shared with libfa.so

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # keep the compiler from emitting packed fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build libfa.so)")
    return path


def _compile(src: str, debug_sync: bool = False) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ("_debugsync" if debug_sync else "") + ".o")
    lang = ["-x", "hip"]
    defs = ["-DFA_DEBUG_SYNC=1"] if debug_sync else []
    cmd = [hipcc(), *HIPCC_FLAGS, *defs, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = [(src, False) for src in SOURCES] + [(src, True) for src in DEBUG_SYNC_SOURCES]
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    fast = objs[:len(SOURCES)]
    _link(fast, OUT)
    dbg = dict(zip(DEBUG_SYNC_SOURCES, objs[len(SOURCES):]))
    _link([dbg.get(src, o) for src, o in zip(SOURCES, fast)], OUT_DEBUG_SYNC)
    if verbose:
        print(f"built {OUT} and {OUT_DEBUG_SYNC}")
    return OUT


if __name__ == "__main__":
    build()
    sys.exit(0)
