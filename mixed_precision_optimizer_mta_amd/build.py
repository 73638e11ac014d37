"""Build libmta.so (the HIP library behind include/mta.h) for gfx950, in-tree.

Flags that carry meaning:
  -ffp-contract=off      no a*b+c -> fma contraction: every float32 operation
                         of the AdamW update is rounded on its own;
  -fhip-fp32-correctly-rounded-divide-sqrt
                         IEEE float32 '/' and sqrtf (HIP's default, stated);
  -fno-gpu-flush-denormals-to-zero
                         denormals are kept (HIP's default, stated);
  -Xclang -target-feature -Xclang -packed-fp32-ops
                         no packed-FP32 (v_pk_*_f32) instructions.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmta.so")
SOURCES = [os.path.join(CSRC, "mta_kernels.hip"),
           os.path.join(CSRC, "mta_host.cpp")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
         "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
         "-fno-gpu-flush-denormals-to-zero",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall"]


def build(verbose=False):
    """Compile libmta.so; always recompiles.  Returns its path."""
    return _compile(LIB, SOURCES, verbose)


def _compile(lib, sources, verbose):
    tmp = lib + ".tmp"
    cmd = [HIPCC, *FLAGS, "-o", tmp, *sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
