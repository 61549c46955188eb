"""Build libkvslot.so (HIP kernels + C ABI) for gfx950 with hipcc.

Usage: python -m decode_attention_slot_amd.build  (or build() from Python).
Every call compiles from source; the library lands next to this file.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkvslot.so")

SOURCES = ["abi.cpp", "slot_mapping.hip", "cache_write.hip", "slot_write.hip", "paged_decode.hip",
           "paged_decode_nc2.hip", "paged_decode_nc4.hip", "lse_merge.hip", "noalloc.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # Packed fp32 VALU ops stay off: scalar fp32 code only.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build(verbose: bool = False) -> str:
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="kvslot_build_") as tmp:
        cmds, objs = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            lang = ["-x", "hip"] if src.endswith(".hip") else []
            cmds.append([cc, *HIPCC_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
            objs.append(obj)
        # one compiler process per source, a few at a time
        with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1, 8)) as pool:
            list(pool.map(lambda c: _run(c, verbose), cmds))
        tmp_lib = os.path.join(tmp, "libkvslot.so")
        _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp_lib], verbose)
        os.replace(tmp_lib, LIB) if _same_fs(tmp_lib, LIB) else shutil.copyfile(tmp_lib, LIB)
    return LIB


def _same_fs(a: str, b: str) -> bool:
    try:
        return os.stat(os.path.dirname(a)).st_dev == os.stat(os.path.dirname(b)).st_dev
    except OSError:
        return False


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


if __name__ == "__main__":
    print(build(verbose=True))
