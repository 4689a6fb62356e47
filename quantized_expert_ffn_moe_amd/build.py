"""Build libmoe.so in-tree for gfx950 with hipcc."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = ["csrc/moe_kernels.hip", "csrc/dense_kernels.hip", "csrc/attn_kernels.hip", "csrc/proj_kernels.hip", "csrc/probe_kernels.hip",
           "csrc/moe_api.cpp", "csrc/dense_api.cpp", "csrc/attn_api.cpp"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         # no packed-FP32 instructions in any generated code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> str:
    out = os.path.join(HERE, "libmoe.so")
    tmp = out + ".tmp"
    cmd = ["hipcc", *FLAGS, "-o", tmp, *[os.path.join(HERE, s) for s in SOURCES]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stderr[-4000:]}")
    if verbose and r.stderr:
        print(r.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
