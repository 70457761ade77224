"""Build libmxq.so for gfx950 in-tree with hipcc.

    python -m mxfp4_microscaled_quantization_amd.build [--verbose]

All HIP sources under csrc/ are compiled into one shared library next to this file.
Packed-FP32 VALU instructions are disabled (-packed-fp32-ops); no fast-math.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmxq.so")
ARCH = "gfx950"

SOURCES = ["mxq_api.hip", "quantize.hip", "gemm.hip", "sqnr.hip"]

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every HIP source into libmxq.so (always rebuilds); returns its path."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, *extra_flags, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass reports the device-only feature flag as unknown: harmless
    noise = ("packed-fp32-ops", "unknown target feature", "-target-feature")
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if ln and not any(n in ln for n in noise)]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
