"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only):
the oracle (oracle/oracle.cpp), the input generator (gen/gen.c) and the C
ABI's host validation (row_wise_normalization_fwd_amd/csrc/api.cpp, its
kernel launches and HIP runtime calls stubbed by tests/san/san_driver.cpp)
are built with g++ / gcc and the sanitizers, and the driver runs them on
small ragged shapes and the ABI's argument matrix. Any report fails the test
(-fno-sanitize-recover: the first one aborts the driver)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1", "-fopenmp"]


def _have(tool):
    return shutil.which(tool) is not None


@pytest.mark.skipif(not (_have("g++") and _have("gcc")), reason="no host compiler")
def test_host_code_under_asan_and_ubsan(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"), "-I",
           os.path.join(ROOT, "row_wise_normalization_fwd_amd", "csrc"),
           "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__"]
    if not os.path.isdir("/opt/rocm/include/hip"):
        pytest.skip("HIP headers not installed")
    objs = []
    jobs = [
        (["gcc", "-std=c11"], os.path.join(ROOT, "gen", "gen.c"), []),
        (["g++", "-std=c++17"], os.path.join(ROOT, "oracle", "oracle.cpp"), []),
        (["g++", "-std=c++17"], os.path.join(ROOT, "row_wise_normalization_fwd_amd", "csrc",
                                             "api.cpp"), inc),
        (["g++", "-std=c++17"], os.path.join(ROOT, "tests", "san", "san_driver.cpp"), inc),
    ]
    procs = []
    for cc, src, extra in jobs:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        procs.append((src, subprocess.Popen(cc + SAN + extra + ["-c", src, "-o", obj],
                                            stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                            text=True)))
        objs.append(obj)
    for src, p in procs:
        out, _ = p.communicate(timeout=300)
        assert p.returncode == 0, f"compiling {src} failed:\n{out}"
    exe = str(tmp_path / "san_driver")
    res = subprocess.run(["g++"] + SAN + objs + ["-o", exe], capture_output=True, text=True,
                         timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    # verify_asan_link_order=0: another preloaded library may come first.
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = res.stdout + res.stderr
    assert res.returncode == 0 and "all checks passed" in res.stdout, out
    assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out
