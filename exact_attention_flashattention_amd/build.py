"""Build libattn.so in-tree with hipcc for gfx950.

Usage: ``python -m exact_attention_flashattention_amd.build`` (or call
``build()``).  Always recompiles.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import time

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libattn.so")

SOURCES = ["attn_abi.hip", "merge_partials.hip", "decode_splitk.hip", "decode_q4.hip", "quantize_q4.hip", "prefill_fwd.hip",
           "calibrate.hip"]

HIPCC_FLAGS = [
    "-std=c++17",
    "-O3",
    "--offload-arch=gfx950",
    "-fPIC",
    "-shared",
    # keep the compiler from forming packed-fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no kernel relies on NaN semantics (masking uses -inf): lets max reductions
    # skip the IEEE quieting of every operand
    "-fno-honor-nans",
    "-Wall",
    "-Wno-unused-function",
]


def hipcc_path() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every HIP source into ``libattn.so`` next to this file."""
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    cmd = [hipcc_path(), *HIPCC_FLAGS, *(extra_flags or []), "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    t0 = time.time()
    proc = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass reports the device-only feature flag as unknown; that line is noise
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (proc.stdout + proc.stderr).splitlines() if noise not in ln]
    if proc.returncode != 0:
        if os.path.exists(tmp):
            os.unlink(tmp)
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(msgs))
    os.replace(tmp, LIB_PATH)
    if verbose:
        if msgs:
            print("\n".join(msgs), file=sys.stderr)
        print(f"built {LIB_PATH} in {time.time() - t0:.1f}s", file=sys.stderr)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
