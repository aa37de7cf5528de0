"""Compile the HIP library ``libattnqat.so`` for gfx950 with hipcc (in-tree)."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libattnqat.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["aq_prep.hip", "aq_attn.hip", "aq_select.hip", "aq_vsa.hip", "aq_mx.hip",
           "aq_noalloc.hip", "aq_api.cpp"]

# Packed fp32 VALU instructions are disabled on purpose: ordinary float code is
# compiled to scalar-lane VALU operations only.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the Attn-QAT library needs ROCm's hipcc to build")


# Machine probes for the benchmark (matrix-core rate and clock), kept out of
# the attention library.
PROBE_SOURCES = ["aq_probe.hip"]
PROBE_PATH = os.path.join(PKG_DIR, "libaq_probe.so")


def _compile(sources, out, verbose):
    srcs = [os.path.join(CSRC, s) for s in sources]
    tmp = out + ".tmp"
    cmd = [hipcc()] + HIP_FLAGS + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if verbose and msgs:
        print(msgs)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile the library (LIB_PATH) and the benchmark's probe library
    (PROBE_PATH); return LIB_PATH."""
    _compile(SOURCES, LIB_PATH, verbose)
    _compile(PROBE_SOURCES, PROBE_PATH, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
