"""Build the gfx950 HIP library ``libxcorr_hip.so`` in-tree with hipcc.

Packed FP32 instructions are disabled for every HIP source (the target
feature ``packed-fp32-ops`` is turned off), so fp32 arithmetic issues as
ordinary single-lane VALU instructions.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libxcorr_hip.so")
SOURCES = ["capi.hip", "ncc_u8.hip", "ncc_u8_mfma.hip", "ncc_u8_mfma32.hip", "ncc_pad.hip", "xcorr_f32.hip", "xcorr_mfma.hip"]
# Issue-rate probes used only by the bench harness (not part of the ABI).
PEAK_LIB = os.path.join(HERE, "libxcorr_peak.so")
PEAK_SOURCES = ["peak_probe.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def build(verbose: bool = False, extra: tuple[str, ...] = (), out: str = LIB) -> str:
    """Compile the correlation library and the bench's peak probes (always rebuilds)."""
    _compile(SOURCES, out, verbose, extra)
    _compile(PEAK_SOURCES, PEAK_LIB, verbose, extra)
    return out


def _compile(sources, out, verbose, extra) -> str:
    srcs = [os.path.join(CSRC, s) for s in sources]
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-shared", f"-I{INCLUDE}", f"-I{CSRC}", *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
