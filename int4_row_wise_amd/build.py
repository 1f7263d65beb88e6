"""Build libqemb.so (the HIP C-ABI library) in-tree for gfx950.

    python -m int4_row_wise_amd.build

hipcc cross-compiles on a machine without a GPU.  Flags: no fast-math and no
floating-point contraction (the quantizer must round exactly as its rules
say), packed-fp32 instructions disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SRC = os.path.join(CSRC, "qemb.hip")  # the translation unit; it includes the csrc/*.inc parts
HEADER = os.path.join(ROOT, "include", "qemb.h")
LIB = os.path.join(HERE, "libqemb.so")
LIB_HASH = LIB + ".srchash"  # source sha256 recorded at build time
# the gather floor (a measurement aid for bench.py, not part of the C ABI)
FLOOR_SRC = os.path.join(CSRC, "gather_floor.hip")
FLOOR_LIB = os.path.join(HERE, "libqemb_floor.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fPIC", "-shared", "-Wall",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    return "hipcc"


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile csrc/qemb.hip into int4_row_wise_amd/libqemb.so."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= max(
            [os.path.getmtime(f) for f in source_files()] + [os.path.getmtime(HEADER)]):
        return LIB
    # the hash of the sources as compiled: taken before the compiler reads
    # them, so an edit made while it runs cannot be recorded for this build
    src_hash = source_sha256()
    # the floor (one small kernel) compiles beside the library
    floor_tmp = FLOOR_LIB + ".tmp%d" % os.getpid()
    floor = subprocess.Popen([hipcc(), *HIPCC_FLAGS, "-o", floor_tmp, FLOOR_SRC], stdout=subprocess.PIPE,
                             stderr=subprocess.STDOUT, text=True)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-o", tmp, SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    floor_out, _ = floor.communicate()
    out = "\n".join(l for l in (r.stdout + floor_out).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0 or floor.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if out.strip() and verbose:
        print(out)
    os.replace(floor_tmp, FLOOR_LIB)
    os.replace(tmp, LIB)
    with open(LIB_HASH, "w") as f:
        f.write(src_hash + "\n")
    return LIB


def source_files() -> list:
    """The kernel sources: qemb.hip, the parts it includes and the gather
    floor, in a fixed order."""
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".inc")))


def source_sha256() -> str:
    """sha256 over the kernel sources the library is built from (each file's
    name and bytes, in sorted order)."""
    import hashlib
    h = hashlib.sha256()
    for path in source_files():
        h.update(os.path.basename(path).encode() + b"\0")
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def built_source_sha256() -> str | None:
    """The source hash recorded when libqemb.so was last built, if any."""
    try:
        with open(LIB_HASH) as f:
            return f.read().strip()
    except OSError:
        return None


def ensure_built() -> str:
    """Build only if no library exists yet (used by tests, smoke and bench)."""
    if os.path.exists(LIB):
        return LIB
    return build(force=True)


if __name__ == "__main__":
    print(build(force=True, verbose="-v" in sys.argv))
