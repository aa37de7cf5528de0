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


# Debug build of the same sources whose kernels fill their LDS arrays with
# NaN before first use (AQ_LDS_POISON): the tests compare it with the release
# library bit for bit, so a read of LDS a kernel never wrote would show.
POISON_PATH = os.path.join(PKG_DIR, "libattnqat_ldspoison.so")

# Machine probes for the benchmark (matrix-core rate and clock), kept out of
# the attention library.
PROBE_SOURCES = ["aq_probe.hip"]
PROBE_PATH = os.path.join(PKG_DIR, "libaq_probe.so")


def _start(sources, out, verbose, extra=()):
    srcs = [os.path.join(CSRC, s) for s in sources]
    tmp = out + ".tmp"
    cmd = [hipcc()] + HIP_FLAGS + list(extra) + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    return proc, tmp, out


def _finish(job, verbose):
    proc, tmp, out = job
    text, _ = proc.communicate()
    msgs = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}) for {out}:\n{msgs}")
    if verbose and msgs:
        print(msgs)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile the library (LIB_PATH), its LDS-poisoning debug twin
    (POISON_PATH) and the benchmark's probe library (PROBE_PATH), in
    parallel; return LIB_PATH."""
    jobs = [_start(SOURCES, LIB_PATH, verbose),
            _start(SOURCES, POISON_PATH, verbose, ["-DAQ_LDS_POISON"]),
            _start(PROBE_SOURCES, PROBE_PATH, verbose)]
    errors = []
    for j in jobs:  # wait for every compiler before reporting a failure
        try:
            _finish(j, verbose)
        except RuntimeError as e:
            errors.append(e)
    if errors:
        raise errors[0]
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
