"""The C-ABI layer built for the host with AddressSanitizer and
UndefinedBehaviorSanitizer (g++, host code only, kernel launchers replaced by
stubs that fail every launch), driven by tests/asan/abi_asan.c: every entry
point refuses bad arguments before any launch, reaches its launch with good
ones without ever touching the caller's device pointers (they point into an
inaccessible mapping), and the split table and workspace sizing stay free of
memory errors and undefined arithmetic over extreme dims.  CPU only."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_gqa_decode_step_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "asan")
HIP_INC = "/opt/rocm/include"


def test_c_abi_under_address_and_ub_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir(HIP_INC):
        pytest.skip("needs g++ and the HIP headers")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-g", "-O1"]
    inc = ["-D__HIP_PLATFORM_AMD__", f"-I{HIP_INC}", f"-I{CSRC}",
           f"-I{os.path.join(ROOT, 'include')}"]
    exe = tmp_path / "abi_asan"
    objs = []
    for src, lang in ((os.path.join(CSRC, "sa_api.cpp"), "c++"),
                      (os.path.join(HERE, "stub_launchers.cpp"), "c++"),
                      (os.path.join(HERE, "abi_asan.c"), "c")):
        obj = tmp_path / (os.path.basename(src) + ".o")
        std = ["-std=c++17"] if lang == "c++" else ["-std=c11", "-D_DEFAULT_SOURCE"]
        r = subprocess.run([gxx, "-x", lang, *std, *san, *inc, "-c", src, "-o", str(obj)],
                           capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, f"compiling {os.path.basename(src)}:\n{r.stderr}"
        objs.append(str(obj))
    r = subprocess.run([gxx, *san, *objs, "-o", str(exe)], capture_output=True, text=True,
                       timeout=300)
    if r.returncode != 0 and "asan" in r.stderr.lower():
        pytest.skip(f"the sanitizer runtimes do not link here:\n{r.stderr[-2000:]}")
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, f"stdout:\n{r.stdout}\nstderr:\n{r.stderr[-6000:]}"
    assert r.stdout.startswith("ok "), r.stdout
