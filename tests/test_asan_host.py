"""Host AddressSanitizer build and run of the C ABI's argument checks and
of the fp64 oracle (tests/asan_check.cpp), without a GPU: the library's
host code and the oracle are compiled with -fsanitize=address (the device
code is not: -Xarch_host), and every C-ABI call made is one that must be
rejected or treated as empty before any HIP call."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_sequence_block_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "asan")


@pytest.mark.slow
@pytest.mark.skipif(shutil.which("hipcc") is None, reason="needs hipcc")
def test_asan_host_checks():
    os.makedirs(OUT, exist_ok=True)
    asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    common = ["--offload-arch=gfx950", "-O3", "-g", "-std=c++17", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    procs = [subprocess.Popen(["hipcc", *common, *asan, "-c", s, "-o",
                               os.path.join(OUT, os.path.basename(s) + ".o")],
                              stderr=subprocess.PIPE, text=True) for s in srcs]
    for p, s in zip(procs, srcs):
        _, err = p.communicate()
        assert p.returncode == 0, f"{s}:\n{err[-3000:]}"
    orc = os.path.join(OUT, "oracle.o")
    r = subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address", "-fopenmp",
                        "-fPIC", "-c", os.path.join(ROOT, "oracle", "blockattn_oracle.c"), "-o",
                        orc], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = os.path.join(OUT, "asan_check")
    drv = os.path.join(OUT, "asan_check.o")
    r = subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-fsanitize=address",
                        "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROOT, "include"),
                        "-I/opt/rocm/include", "-c", os.path.join(ROOT, "tests", "asan_check.cpp"),
                        "-o", drv], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    objs = [os.path.join(OUT, os.path.basename(s) + ".o") for s in srcs]
    r = subprocess.run(["g++", "-fsanitize=address", drv, *objs, orc, "-fopenmp",
                        "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", OMP_NUM_THREADS="2")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "PASSED (0 failures)" in r.stdout
