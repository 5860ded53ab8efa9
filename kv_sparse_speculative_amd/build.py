"""Build libkvss.so (the HIP kernels and their C ABI) in-tree for gfx950 with hipcc."""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvss.so")
SOURCES = ["api.hip", "attn_mfma.hip", "attn_simple.hip", "merge.hip", "snapkv.hip", "snapkv_mfma.hip",
           "accept.hip", "streaming.hip", "stream.hip", "cache.hip", "sample.hip", "philox.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core results land in ordinary VGPRs (no accumulator-register copies)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose=False):
    """Compile every HIP source into kv_sparse_speculative_amd/libkvss.so (always rebuilds)."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           "-o", tmp, *[os.path.join(CSRC, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libkvss.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
