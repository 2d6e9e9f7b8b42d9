"""Build libmsa.so in-tree with hipcc for gfx950.

    python -m block_sparse_paged_query_amd.build     # or build() from Python
    python -m block_sparse_paged_query_amd.build --sanitize   # host ASan/UBSan copy

Every ``csrc/*.hip`` file is compiled to an object (in parallel), then linked
into ``block_sparse_paged_query_amd/libmsa.so``.  Packed fp32 instructions are
disabled for the device code (``-packed-fp32-ops``); the host pass warns that
it does not know that feature, which is harmless.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmsa.so")
OBJ_DIR = os.path.join(PKG, "_build")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# Host-side sanitizer build (CPU testing of the argument validation only; the
# device code is built as usual): an instrumented copy of the library in its
# own folder, loaded with the ASan runtime preloaded.
SAN_DIR = os.path.join(PKG, "_build_san")
SAN_LIB = os.path.join(SAN_DIR, "libmsa.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(SAN_DIR if sanitize else OBJ_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *(SAN_FLAGS if sanitize else []), "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every HIP source and link libmsa.so; returns the library path.
    sanitize=True builds the host-instrumented copy (SAN_LIB) instead."""
    out_dir, lib = (SAN_DIR, SAN_LIB) if sanitize else (OBJ_DIR, LIB)
    os.makedirs(out_dir, exist_ok=True)
    sources = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    jobs = min(len(sources), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(max_workers=max(jobs, 1)) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), sources))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *(SAN_FLAGS if sanitize else []), "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib} from {len(sources)} sources")
    return lib


if __name__ == "__main__":
    build(verbose=True, sanitize="--sanitize" in sys.argv[1:])
    sys.exit(0)
