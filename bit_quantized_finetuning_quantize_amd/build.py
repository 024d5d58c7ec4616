"""Build the HIP library (libqlora.so) for gfx950 with hipcc.

Run as `python bit_quantized_finetuning_quantize_amd/build.py` (by path, so
that the package, which loads the library, is not imported first) or call
`build()`. The library is written next to this file, in-tree.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqlora.so")
SOURCES = ["quant.hip", "gemv.hip", "linear.hip", "adamw.hip", "dropout.hip", "noalloc.hip", "api.cpp"]
ARCH = "gfx950"

FLAGS = [
    "-O3",
    "-std=c++20",
    "-fPIC",
    "-shared",
    f"--offload-arch={ARCH}",
    # packed float32 VALU forms are kept out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def build(verbose=False):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc] + FLAGS + ["-I", CSRC, "-o", tmp] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libqlora.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
