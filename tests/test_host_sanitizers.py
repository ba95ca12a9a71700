"""The host half of the library under AddressSanitizer and UndefinedBehaviorSanitizer,
and under ThreadSanitizer.

abi.cpp and plan.cpp (argument checks, decode / ragged / cascade plans,
workspace layouts) are built by the host compiler with -fsanitize=address,undefined
and stub kernel launchers, then the CPU tests that drive them through the C ABI
run against that build in a child process. A second build with
-fsanitize=thread runs the test that calls the host side from eight threads at
once. Any sanitizer report fails the test.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_20_amd", "csrc")
ROCM = "/opt/rocm"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
DRIVEN = ["tests/test_abi_cpu.py", "tests/test_ragged_cpu.py", "tests/test_cascade_cpu.py"]


def _runtime(name):
    p = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _host_build(d, name, flags):
    if shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")):
        pytest.skip("g++ or the HIP headers are missing")
    lib = str(d / name)
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-shared", "-fPIC", *flags, "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "abi.cpp"), os.path.join(CSRC, "plan.cpp"),
           os.path.join(ROOT, "tests", "host_sanitize", "launch_stubs.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"sanitizer build failed:\n{' '.join(cmd)}\n{r.stderr[-4000:]}"
    return lib


@pytest.fixture(scope="module")
def san_lib(tmp_path_factory):
    return _host_build(tmp_path_factory.mktemp("hostsan"), "libfa_host_san.so", SAN)


def test_host_code_under_asan_ubsan(san_lib, tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("sanitizer runtimes not found")
    logs = tmp_path / "reports"
    logs.mkdir()
    env = dict(os.environ)
    # Reports go to files (pytest's capture of fd 2 would hide a report from a
    # process the sanitizer ends).
    env.update(FA_LIBRARY=san_lib, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS=f"detect_leaks=0:allocator_may_return_null=1:log_path={logs}/asan",
               UBSAN_OPTIONS=f"print_stacktrace=1:halt_on_error=1:log_path={logs}/ubsan",
               HIP_VISIBLE_DEVICES="")
    r = subprocess.run([sys.executable, "-m", "pytest", *DRIVEN, "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    out = r.stdout + r.stderr
    reports = sorted(logs.iterdir())
    assert not reports, "sanitizer report:\n" + "\n".join(p.read_text()[-4000:] for p in reports)
    assert r.returncode == 0, f"CPU tests failed against the sanitizer build:\n{out[-6000:]}"
    assert " passed" in out
    # the child really loaded the sanitizer build
    chk = subprocess.run([sys.executable, "-c", "import exact_attention_20_amd as fa; fa.load(); print(fa.lib_path())"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert chk.stdout.strip().endswith("libfa_host_san.so"), chk.stdout + chk.stderr


def test_host_code_under_tsan(tmp_path):
    tsan = _runtime("libtsan.so")
    if tsan is None:
        pytest.skip("ThreadSanitizer runtime not found")
    lib = _host_build(tmp_path, "libfa_host_tsan.so", ["-fsanitize=thread", "-fno-omit-frame-pointer"])
    logs = tmp_path / "reports"
    logs.mkdir()
    env = dict(os.environ)
    env.update(FA_LIBRARY=lib, LD_PRELOAD=tsan, TSAN_OPTIONS=f"log_path={logs}/tsan", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi_cpu.py", "-q", "-x", "-m", "not gpu",
                        "-k", "many_threads", "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    out = r.stdout + r.stderr
    reports = sorted(logs.iterdir())
    assert not reports, "sanitizer report:\n" + "\n".join(p.read_text()[-4000:] for p in reports)
    assert r.returncode == 0 and "1 passed" in out, f"threaded test failed against the TSan build:\n{out[-6000:]}"
