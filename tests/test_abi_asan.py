"""Host-side argument validation of the C ABI under AddressSanitizer.

abi.hip (the C ABI layer) is rebuilt with ASan on the host side only
(-Xarch_host; the device code is unchanged), linked with the other objects
of the regular build into a throw-away liblcp, and driven by
tests/asan_driver.c: every entry point is called with defective arguments
(null, misaligned or undersized buffers, bad shapes and options) and must
return its error code before any HIP call, with no ASan report. Needs the
objects of learnable_channel_permutation_amd/build.py under _build/; no GPU.
"""
import os
import shlex
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OBJ = os.path.join(ROOT, "_build")
CSRC = os.path.join(ROOT, "learnable_channel_permutation_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/lib/llvm/bin/clang"
HOST_ASAN = "-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer"


def test_abi_validation_under_asan(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("ROCm compilers not available")
    objs = sorted(os.path.join(OBJ, f) for f in os.listdir(OBJ)) if os.path.isdir(OBJ) else []
    objs = [o for o in objs if o.endswith(".o") and os.path.basename(o) != "abi.o"]
    if not objs:
        pytest.skip("no build objects (run learnable_channel_permutation_amd/build.py)")
    abi_o = str(tmp_path / "abi_asan.o")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + shlex.split(HOST_ASAN) + \
          ["-c", os.path.join(CSRC, "abi.hip"), "-o", abi_o]
    p = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert p.returncode == 0, p.stderr
    lib = str(tmp_path / "liblcp_asan.so")
    p = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib, abi_o] + objs,
                       capture_output=True, text=True, timeout=600)
    assert p.returncode == 0, p.stderr
    exe = str(tmp_path / "asan_driver")
    p = subprocess.run([CLANG, "-std=c99", "-Wall", "-Wextra", "-Werror", "-fsanitize=address",
                        "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
                        os.path.join(ROOT, "tests", "asan_driver.c"), "-L", str(tmp_path), "-llcp_asan",
                        "-Wl,-rpath," + str(tmp_path), "-o", exe], capture_output=True, text=True, timeout=600)
    assert p.returncode == 0, p.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr[-4000:])
    assert r.stdout.strip().startswith("ok "), r.stdout
    assert "AddressSanitizer" not in r.stderr
