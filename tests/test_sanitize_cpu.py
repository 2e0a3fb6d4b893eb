"""The CPU oracle and the library's host code (argument checks, layouts,
split plans, workgroup roles, launch arguments) built with the address and
undefined-behaviour sanitizers and driven through their entry points
(tests/sanitize/drive.py).  The host code is linked against stand-in kernel
launchers (tests/sanitize/stub_kernels.cpp) that check the arguments each
launch would get, so valid calls run end to end on the CPU.  Any sanitizer
finding aborts the driver."""
import os
import pathlib
import shutil
import subprocess
import sys

import pytest

from oracle import CFLAGS as ORACLE_CFLAGS

ROOT = pathlib.Path(__file__).resolve().parents[1]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"


@pytest.mark.timeout(900)
def test_oracle_and_host_code_under_sanitizers(tmp_path):
    if not (shutil.which("gcc") and shutil.which("g++")):
        pytest.skip("no host compiler")
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                             text=True).stdout.strip()
    if not os.path.isabs(libasan) or not os.path.exists(libasan):
        pytest.skip("no address-sanitizer runtime")
    oracle_so = tmp_path / "liboracle_san.so"
    flags = [f for f in ORACLE_CFLAGS if f != "-O2"]
    _run(["gcc", *flags, *SAN, str(ROOT / "oracle" / "loopvq_oracle.c"), "-o", str(oracle_so), "-lm"])
    host_so = tmp_path / "libloopvq_host_san.so"
    _run(["g++", "-std=c++17", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
          f"-I{ROOT / 'include'}", f"-I{ROOT / 'sub_bit_vq_amd' / 'csrc'}", *SAN, "-Wl,--no-undefined",
          str(ROOT / "sub_bit_vq_amd" / "csrc" / "loopvq_host.cpp"),
          str(ROOT / "tests" / "sanitize" / "stub_kernels.cpp"), "-o", str(host_so)])
    env = dict(os.environ, LD_PRELOAD=libasan, OMP_NUM_THREADS="2",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, str(ROOT / "tests" / "sanitize" / "drive.py"), str(oracle_so),
                        str(host_so)], capture_output=True, text=True, env=env, timeout=800)
    assert r.returncode == 0, f"{r.stdout[-3000:]}\n{r.stderr[-6000:]}"
    assert "sanitized drive ok" in r.stdout
