"""The oracle and the host logic of libmta under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

tests/c/san_oracle.c drives every function of oracle/mta_oracle.c over edge
sizes and type combinations on buffers of exactly their contract's size;
tests/c/san_host.c drives mta_host.cpp (validation, tile planning, overlap
checks, scalar preparation, error reporting) through include/mta.h with no
device, its kernel launchers replaced by stubs that must never be reached
(tests/c/san_stubs.cpp).  Both are built with gcc / g++ (host code only) and
must exit 0 with no sanitizer report.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
C = os.path.join(ROOT, "tests", "c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stderr[-4000:]}"


@pytest.fixture(scope="module")
def _compilers():
    for tool in ("gcc", "g++"):
        if shutil.which(tool) is None:
            pytest.skip(f"{tool} not found")


def test_oracle_under_sanitizers(tmp_path, _compilers):
    exe = str(tmp_path / "san_oracle")
    _run(["gcc", "-std=c11", *SAN, "-ffp-contract=off", "-o", exe,
          os.path.join(C, "san_oracle.c"),
          os.path.join(ROOT, "oracle", "mta_oracle.c"), "-lm"], tmp_path)
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "clean" in r.stdout


def test_host_library_under_sanitizers(tmp_path, _compilers):
    if not os.path.exists(os.path.join(ROCM, "include", "hip",
                                       "hip_runtime.h")):
        pytest.skip("HIP headers not found")
    hip = ["-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include"]
    objs = []
    for src, lang in (
            (os.path.join(ROOT, "mixed_precision_optimizer_mta_amd", "csrc",
                          "mta_host.cpp"), "c++"),
            (os.path.join(C, "san_stubs.cpp"), "c++"),
            (os.path.join(C, "san_host.c"), "c")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        cc = ["g++", "-std=c++17"] if lang == "c++" else ["gcc", "-std=c11"]
        _run([*cc, *SAN, *hip, f"-I{ROOT}/include", "-c", "-o", obj, src],
             tmp_path)
        objs.append(obj)
    exe = str(tmp_path / "san_host")
    _run(["g++", *SAN, "-o", exe, *objs, f"-L{ROCM}/lib", "-lamdhip64",
          f"-Wl,-rpath,{ROCM}/lib"], tmp_path)
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "clean" in r.stdout
