"""Build the PBSA HIP library (libpbsa.so) in-tree for gfx950 with hipcc.

Usage: python -m block_sparse_attention_15_amd.build [--force] [--lds-check]
(or build() from Python).
Compiles every .hip file under csrc/ to an object, then links one shared
library next to this file.  Objects are rebuilt only when their source or a
header changed, unless force=True.
"""
from __future__ import annotations

import glob
import hashlib
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build", "obj")
LIB = os.path.join(HERE, "libpbsa.so")
# The LDS-race check build: the same sources with every LDS-bound load waited
# for at once and every step barrier draining all loads (PBSA_LDS_RACE_CHECK);
# its outputs must equal the product library's bit for bit.  Test use only.
LIB_LDS_CHECK = os.path.join(HERE, "libpbsa_ldscheck.so")

ARCH = os.environ.get("PBSA_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-honor-nans",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable", "-Wno-unused-result",
    "-I", INCLUDE, "-I", CSRC,
]


def _headers():
    return glob.glob(os.path.join(CSRC, "*.h")) + glob.glob(os.path.join(INCLUDE, "*.h"))


def _compile(src: str, force: bool, objdir: str = OBJDIR, extra=()) -> str:
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    if not force and os.path.exists(obj):
        t = os.path.getmtime(obj)
        if all(os.path.getmtime(d) < t for d in [src] + _headers()):
            return obj
    cmd = [HIPCC] + FLAGS + list(extra) + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def source_digest() -> str:
    """SHA-256 over the kernel sources, headers and code-generation flags (not
    paths), identifying the compiled kernels that a profile was taken on."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + _headers(), key=os.path.basename)
    for f in files:
        h.update(os.path.basename(f).encode() + b"\0")
        with open(f, "rb") as fh:
            h.update(fh.read())
    h.update(" ".join(x for x in FLAGS if x not in (INCLUDE, CSRC)).encode())
    return h.hexdigest()[:16]


def build(force: bool = True, verbose: bool = False, lds_check: bool = False) -> str:
    """Build libpbsa.so, or with lds_check the LDS-race check library."""
    objdir = OBJDIR + ("_ldscheck" if lds_check else "")
    lib = LIB_LDS_CHECK if lds_check else LIB
    extra = ["-DPBSA_LDS_RACE_CHECK=1"] if lds_check else []
    os.makedirs(objdir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, force, objdir, extra), srcs))
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(force="--force" in sys.argv, verbose=True, lds_check="--lds-check" in sys.argv)
