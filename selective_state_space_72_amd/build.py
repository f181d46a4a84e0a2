"""Build libmambascan.so (HIP, gfx950) in-tree.

    python -m selective_state_space_72_amd.build

Each ``csrc/*.hip`` file is compiled to an object in ``_build/`` (in parallel)
and linked into ``selective_state_space_72_amd/libmambascan.so``.  Device code
is compiled without packed-FP32 instructions.

A digest of the sources (``csrc/*.hip``, ``csrc/*.h``, ``include/*.h``) and of the
compiler flags is written next to the library; ``is_built()`` is true only while it
matches, so ``ensure_built()`` rebuilds a library that is older than its sources.
"""

from __future__ import annotations

import concurrent.futures
import glob
import hashlib
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIBRARY = os.path.join(PKG, "libmambascan.so")
DIGEST_FILE = LIBRARY + ".digest"
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", f"--offload-arch={ARCH}", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def source_digest() -> str:
    """sha256 over the compiler, flags and every source and header the library is built from."""
    h = hashlib.sha256()
    h.update(" ".join([HIPCC, ARCH, *FLAGS]).encode())
    files = (sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + sorted(glob.glob(os.path.join(CSRC, "*.h")))
             + sorted(glob.glob(os.path.join(INCLUDE, "*.h"))))
    for f in files:
        h.update(os.path.relpath(f, ROOT).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(line for line in r.stderr.splitlines()
                     if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{errs}")
    if errs.strip():
        print(errs, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    digest = source_digest()
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIBRARY + ".tmp"
    subprocess.run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp],
                   check=True)
    os.replace(tmp, LIBRARY)
    with open(DIGEST_FILE, "w") as fh:
        fh.write(digest + "\n")
    if verbose:
        print(f"built {LIBRARY}")
    return LIBRARY


def is_built() -> bool:
    """True if the library exists and was built from the current sources and flags."""
    if not (os.path.exists(LIBRARY) and os.path.exists(DIGEST_FILE)):
        return False
    with open(DIGEST_FILE) as fh:
        return fh.read().strip() == source_digest()


def ensure_built(verbose: bool = True) -> str:
    """Build the library unless an up-to-date one is in place."""
    if not is_built():
        build(verbose)
    return LIBRARY


if __name__ == "__main__":
    build()
