"""Build libnested_linear.so (gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libnested_linear.so")
SOURCES = ["nl_kernels.hip", "nl_api.hip", "nl_encode.hip", "nl_w4w8.hip", "nl_tree.hip", "nl_kv.hip"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
    # packed fp32 VALU ops stay off: the compiler's own scalar code is used
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the epilogue reads them every group
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def build(verbose: bool = False) -> str:
    """Compile every HIP source into bit_nested_quantized_amd/libnested_linear.so."""
    tmp = LIB + ".tmp"
    cmd = ["hipcc", *FLAGS, "-o", tmp, *[os.path.join(CSRC, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
