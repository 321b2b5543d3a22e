"""Build the HIP library (libgptq_mi355x.so) in-tree for gfx950 with hipcc.

Usage: python -m post_weight_quantization_gptq_amd.build_lib
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgptq_mi355x.so")
SOURCES = ["syrk.hip", "factor.hip", "sweep.hip", "lora.hip", "round2d.hip", "qronos.hip", "deploy.hip", "planner.cpp", "api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fvisibility=hidden",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-ffp-contract=on",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def build(verbose: bool = False) -> str:
    """Compile every source into one shared library; returns its path."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC] + FLAGS + ["-x", "hip"] + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building %s" % LIB)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
