"""Build libgdn.so (the HIP kernels and the C ABI of include/gdn.h) and
libgdn_ceiling.so (the measurement kernels of include/gdn_ceiling.h) for gfx950.

Run as `python -m linear_attention_sequence_amd.build` or call build(). The
libraries are written next to this file, with build_info.json (the commit and
source digest they were built from); nothing is installed elsewhere.
"""
from __future__ import annotations

import hashlib
import json
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libgdn.so")
SOURCES = ["gdn_api.cpp", "gdn_recurrent.hip", "gdn_conv.hip", "gdn_prefill.hip", "gdn_prefill_mfma.hip",
           "gdn_noalloc.hip"]
CEILING_LIB = os.path.join(HERE, "libgdn_ceiling.so")
CEILING_SOURCES = ["gdn_ceiling.hip"]
# the MFMA throughput loops keep their accumulators in VGPRs: with AGPR accumulators the
# register allocator moved the 16x16x32 chains between registers every iteration
CEILING_FLAGS = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
BUILD_INFO = os.path.join(HERE, "build_info.json")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    # packed fp32 instructions stay off: the kernels are written for scalar fp32
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def source_digest() -> str:
    """SHA-256 (16 hex digits) over every source and header the libraries are built from."""
    h = hashlib.sha256()
    files = sorted(os.listdir(CSRC)) + sorted(os.listdir(INCLUDE))
    for name in files:
        path = os.path.join(CSRC if os.path.exists(os.path.join(CSRC, name)) else INCLUDE, name)
        if os.path.isfile(path) and name.endswith((".hip", ".cpp", ".hpp", ".h")):
            h.update(name.encode())
            with open(path, "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def _git_commit() -> str | None:
    try:
        out = subprocess.run(["git", "-C", ROOT, "describe", "--always", "--dirty", "--abbrev=12"],
                             capture_output=True, text=True, timeout=10)
        return out.stdout.strip() or None
    except (OSError, subprocess.SubprocessError):
        return None


def _compile(sources, out, verbose, extra=()):
    srcs = [os.path.join(CSRC, s) for s in sources]
    tmp = out + ".tmp"
    # only the C ABI is exported (csrc/exports.map)
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, *srcs,
           "-Wl,--version-script=" + os.path.join(CSRC, "exports.map"), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile libgdn.so and libgdn_ceiling.so (always recompiles)."""
    _compile(SOURCES, LIB, verbose)
    _compile(CEILING_SOURCES, CEILING_LIB, verbose, CEILING_FLAGS)
    with open(BUILD_INFO, "w") as f:
        json.dump({"commit": _git_commit(), "source_digest": source_digest(),
                   "hipcc_flags": " ".join(HIPCC_FLAGS)}, f)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
