"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two executables are built with ``-fsanitize=address,undefined,
float-cast-overflow -fno-sanitize-recover=all`` and run:

* the C-ABI layer of the library (``dcnv4_api.cpp``, ``fdattn_api.cpp``,
  compiled by g++ as plain host C++) against the launch stand-ins of
  ``tests/sanitize/host_fakes.cpp``, driven through thousands of seeded valid
  and invalid calls (``tests/sanitize/host_driver.cpp``): every status must be
  a documented one, every accepted call must launch exactly its N images,
  every launch must stay inside the caller's tensors and fit 31-bit offsets;
* both CPU oracles on small problems whose sampling locations include NaN,
  +-inf, +-1e30 and the exact borders (``tests/sanitize/oracle_driver.c``).

The same commands, for use by hand, are printed by ``python -m
tests.test_host_sanitizers``.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "dynamic_sparse_vision_amd", "csrc")
SANITIZE = ["-O1", "-g", "-fno-omit-frame-pointer",
            "-fsanitize=address,undefined,float-cast-overflow", "-fno-sanitize-recover=all"]
ENV = {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0:halt_on_error=1",
       "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def host_command(out):
    return ["g++", "-std=c++17", *SANITIZE, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
            "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, "-I" + SAN,
            os.path.join(CSRC, "dcnv4_api.cpp"), os.path.join(CSRC, "fdattn_api.cpp"),
            os.path.join(SAN, "host_fakes.cpp"), os.path.join(SAN, "host_driver.cpp"), "-o", out]


def oracle_command(out):
    return ["gcc", "-std=c11", *SANITIZE, "-ffp-contract=off",
            os.path.join(ROOT, "oracle", "dcnv4_oracle.c"), os.path.join(ROOT, "oracle", "fdattn_oracle.c"),
            os.path.join(SAN, "oracle_driver.c"), "-o", out, "-lm"]


def _build_and_run(cmd, exe):
    if shutil.which(cmd[0]) is None:
        pytest.skip(cmd[0] + " not found")
    if not os.path.exists("/opt/rocm/include/hip/hip_runtime.h") and cmd[0] == "g++":
        pytest.skip("HIP headers not found")
    subprocess.run(cmd, check=True, timeout=300)
    env = dict(os.environ, **ENV)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert r.stdout.startswith("ok "), r.stdout
    return r.stdout


def test_c_abi_layer_under_asan_ubsan(tmp_path):
    out = _build_and_run(host_command(str(tmp_path / "host_driver")), str(tmp_path / "host_driver"))
    calls, accepted = int(out.split()[1]), int(out.split()[3])
    assert calls > 10000 and accepted > 3000, out


def test_oracles_under_asan_ubsan(tmp_path):
    out = _build_and_run(oracle_command(str(tmp_path / "oracle_driver")), str(tmp_path / "oracle_driver"))
    assert int(out.split()[1]) > 5000, out


if __name__ == "__main__":
    exe = sys.argv[1] if len(sys.argv) > 1 else "/tmp"
    print(" ".join(host_command(os.path.join(exe, "host_driver"))))
    print(" ".join(oracle_command(os.path.join(exe, "oracle_driver"))))
