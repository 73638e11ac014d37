"""Build tests/c/abi_demo: a C program linked against libmta.so and the HIP
runtime, compiled by gcc from include/mta.h alone (the C boundary, no C++)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "mixed_precision_optimizer_mta_amd")
EXE = os.path.join(HERE, "abi_demo")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose=False):
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra",
           "-D__HIP_PLATFORM_AMD__", f"-I{ROOT}/include", f"-I{ROCM}/include",
           os.path.join(HERE, "abi_demo.c"), "-o", EXE + ".tmp",
           f"-L{PKG}", "-lmta", f"-L{ROCM}/lib", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../mixed_precision_optimizer_mta_amd",
           f"-Wl,-rpath,{ROCM}/lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed ({r.returncode}):\n{r.stderr}")
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build(verbose=True))
