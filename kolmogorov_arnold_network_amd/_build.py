"""Builds the HIP library ``libkan_mi355x.so`` in-tree with hipcc for gfx950.

Each source is compiled to its own object in parallel (no device code crosses
a translation unit), then the objects are linked into the shared library.
"""

import os
import shutil
import subprocess
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(REPO_DIR, "include")
LIB_NAME = "libkan_mi355x.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["kan_api.cpp", "kan_plan.cpp", "kan_gather.hip", "kan_grouped.hip", "kan_mfma.hip", "kan_static.hip"]

# -packed-fp32-ops off: the compiler must not form packed float32 ALU ops.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (needs ROCm)")


def _filter(text):
    return "\n".join(l for l in text.splitlines()
                     if "packed-fp32-ops' is not a recognized feature" not in l)


def build_library(verbose=False):
    """Compile every source for gfx950 into ``LIB_PATH`` (always recompiles)."""
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="kanbuild") as tmpdir:
        jobs = []
        for s in SOURCES:
            obj = os.path.join(tmpdir, s + ".o")
            cmd = [cc] + HIPCC_FLAGS + ["-I" + INCLUDE, "-I" + CSRC, "-c", "-o", obj,
                                        os.path.join(CSRC, s)]
            jobs.append((cmd, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                    stderr=subprocess.STDOUT, text=True)))
        msgs, failed = [], []
        for cmd, obj, proc in jobs:
            out, _ = proc.communicate()
            out = _filter(out)
            if out.strip():
                msgs.append(out)
            if proc.returncode != 0:
                failed.append(" ".join(cmd) + "\n" + out)
        if failed:
            raise RuntimeError("hipcc failed:\n" + "\n\n".join(failed))
        tmp = LIB_PATH + ".tmp"
        cmd = [cc] + HIPCC_FLAGS + ["-shared", "-o", tmp] + [obj for _, obj, _ in jobs]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("link failed:\n" + " ".join(cmd) + "\n" + _filter(res.stdout + res.stderr))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose=True))
