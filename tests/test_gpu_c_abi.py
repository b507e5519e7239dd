"""The GPU entry points from plain C: tests/c/ns_abi_gpu.c is compiled as C99
with gcc against include/ns.h and HIP's C runtime API (-Wall -Wextra
-pedantic -Werror; HIP's headers come in as system headers, which are not
pedantic-clean C), linked to the built libnsq.so and run as a child process.
It runs ns_orthogonalize_batched on a matrix whose singular values are all
equal, against the closed form, and a pack/unpack round trip through a route
plan, bit for bit."""

import os
import shutil
import subprocess

import pytest

import newton_schulz_quintic_amd as nsq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_c99_caller_of_the_gpu_entry_points(tmp_path):
    if not os.path.exists(nsq.LIB_PATH):
        pytest.fail("libnsq.so not built")
    lib_dir = os.path.dirname(nsq.LIB_PATH)
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    rocm_lib = os.path.join(rocm, "lib")
    exe = str(tmp_path / "ns_abi_gpu")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-isystem", os.path.join(rocm, "include"),
           os.path.join(ROOT, "tests", "c", "ns_abi_gpu.c"),
           "-L", lib_dir, "-lnsq", "-L", rocm_lib, "-lamdhip64", "-lm",
           f"-Wl,-rpath,{lib_dir}", f"-Wl,-rpath,{rocm_lib}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    print("running", exe, flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=90)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout, r.stderr)
