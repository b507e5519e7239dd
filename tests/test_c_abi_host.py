"""The C ABI from plain C: tests/c/ns_abi_host.c is compiled as C99 with gcc
against include/ns.h (-Wall -Wextra -pedantic -Werror), linked to the built
libnsq.so and run. It calls the host-only entry points (planner, route plans,
waves, workspace sizes, errors) and checks values worked by hand from the
header's contracts. No GPU is needed."""

import os
import shutil
import subprocess

import pytest

import newton_schulz_quintic_amd as nsq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_c99_caller_of_the_host_entry_points(tmp_path):
    if not os.path.exists(nsq.LIB_PATH):
        pytest.skip("libnsq.so not built")
    lib_dir = os.path.dirname(nsq.LIB_PATH)
    rocm_lib = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib")
    exe = str(tmp_path / "ns_abi_host")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "ns_abi_host.c"),
           "-L", lib_dir, "-lnsq", f"-Wl,-rpath,{lib_dir}", f"-Wl,-rpath-link,{rocm_lib}",
           f"-Wl,-rpath,{rocm_lib}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stderr
