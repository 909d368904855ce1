"""Build libnested_linear.so (gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libnested_linear.so")
SOURCES = ["nl_kernels.hip", "nl_fwd.hip", "nl_api.hip", "nl_encode.hip", "nl_w4w8.hip", "nl_tree.hip", "nl_kv.hip", "nl_stream.hip"]
FLAGS_C = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # packed fp32 VALU ops stay off: the compiler's own scalar code is used
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the epilogue reads them every group
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    return r.returncode, err


def build(verbose: bool = False) -> str:
    """Compile every HIP source (in parallel, one object each) and link
    bit_nested_quantized_amd/libnested_linear.so."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    jobs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        jobs.append((["hipcc", *FLAGS_C, "-c", "-o", obj, os.path.join(CSRC, src)], obj))
    workers = max(1, min(len(jobs), os.cpu_count() or 1, 8))
    with ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(lambda j: _run(j[0]), jobs))
    for (cmd, _), (rc, err) in zip(jobs, results):
        if verbose:
            print(" ".join(cmd), flush=True)
        if rc != 0:
            raise RuntimeError("hipcc failed:\n" + err)
        if verbose and err:
            print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    link = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *[o for _, o in jobs]]
    rc, err = _run(link)
    if verbose:
        print(" ".join(link), flush=True)
    if rc != 0:
        raise RuntimeError("link failed:\n" + err)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
