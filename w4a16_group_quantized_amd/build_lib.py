"""Build libmoe_w4a16.so for gfx950 with hipcc, in-tree.

Run as ``python -m w4a16_group_quantized_amd.build_lib`` or through
``__graft_entry__.build()``.  Always recompiles.
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(os.path.dirname(PKG_DIR), "include")
LIB_NAME = "libmoe_w4a16.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ["abi.hip", "plan.hip", "route.hip", "permute.hip", "route_permute.hip",
           "router_gate.hip", "ffn_decode.hip", "ffn_prefill.hip", "combine.hip"]
ARCH = "gfx950"

FLAGS = [
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    f"--offload-arch={ARCH}",
    "-Wall",
    "-Wno-unused-function",
    # keep the compiler from forming packed fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-instruction results in ordinary vector registers, which the fp32
    # scaling reads directly (no accumulation-register copies)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
