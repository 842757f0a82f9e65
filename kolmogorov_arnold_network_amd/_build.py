"""Builds the HIP library ``libkan_mi355x.so`` in-tree with hipcc for gfx950."""

import os
import shutil
import subprocess

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(REPO_DIR, "include")
LIB_NAME = "libkan_mi355x.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["kan_api.cpp", "kan_gather.hip", "kan_grouped.hip", "kan_mfma.hip"]

# -packed-fp32-ops off: the compiler must not form packed float32 ALU ops.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (needs ROCm)")


def build_library(verbose=False):
    """Compile every source for gfx950 into ``LIB_PATH`` (always recompiles)."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc()] + HIPCC_FLAGS + ["-I" + INCLUDE, "-I" + CSRC, "-o", tmp] + srcs
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                     if "packed-fp32-ops' is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + msgs)
    if verbose and msgs.strip():
        print(msgs)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose=True))
