"""The CPU sanitizer job: the host code of the library (kda_api.cpp: the
C ABI's argument and alias checks, workspace planning and argument packing,
linked with the host-only stand-ins of tests/sanitize/host_stubs.cpp instead
of the kernel launchers) and the fp64 oracle are built with the address and
undefined-behaviour sanitizers (undefined behaviour aborts), and the ABI
tests, a run of valid calls through every host path, and the oracle's pins
(including the planted-slip builds) run against those builds in a child
process with the sanitizer runtimes preloaded.  A planted heap overflow
checks that the job does catch one.  CPU only; needs g++ and its sanitizer
runtimes."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


pytestmark = pytest.mark.skipif(shutil.which("g++") is None or not _runtime("libasan.so")
                                or not _runtime("libubsan.so"), reason="needs g++ and its sanitizer runtimes")


def _env(extra):
    env = dict(os.environ)
    env["LD_PRELOAD"] = f"{_runtime('libasan.so')}:{_runtime('libubsan.so')}"
    # Python and torch keep memory until exit by design: leak reports are off
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env.update(extra)
    return env


def _pytest(files, env):
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", *files],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    return out


@pytest.fixture(scope="module")
def host_lib(tmp_path_factory):
    d = tmp_path_factory.mktemp("san")
    lib = str(d / "libkda_host_san.so")
    cmd = ["g++", "-std=c++17", "-O1", "-fPIC", "-shared", *SAN, "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "linear_attention_kda_amd", "csrc"),
           "-o", lib, os.path.join(ROOT, "linear_attention_kda_amd", "csrc", "kda_api.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "host_stubs.cpp")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return lib


def test_abi_host_code_under_sanitizers(host_lib):
    out = _pytest(["tests/test_abi.py", "tests/sanitize/host_paths_stub.py"], _env({"KDA_LIBRARY": host_lib}))
    assert " passed" in out and "skipped" not in out


def test_oracle_under_sanitizers(tmp_path):
    out = _pytest(["tests/test_oracle_pins.py", "tests/test_compare.py"],
                  _env({"KDA_ORACLE_LIB": str(tmp_path / "libkda_oracle.so"),
                        "KDA_ORACLE_CFLAGS": " ".join(SAN)}))
    assert " passed" in out


def test_the_job_catches_a_planted_overflow(tmp_path):
    # built and run the way the oracle is: gcc with the same flags, loaded
    # into a process with the runtimes preloaded
    src = tmp_path / "bad.c"
    src.write_text("#include <stdlib.h>\nint main(void){volatile int *p = malloc(4 * sizeof(int));"
                   "p[4] = 1; free((void*)p); return 0;}\n")
    exe = str(tmp_path / "bad")
    subprocess.run(["gcc", *SAN, "-o", exe, str(src)], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, env=_env({}))
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr
