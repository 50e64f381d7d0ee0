"""The boundary from plain C: include/kpool.h compiles as ISO C11 with every
warning an error, and a C program linked against libkpool.so gets the
version, sizes, status strings and argument validation of the library
without a GPU (no call here reaches a kernel launch)."""
import os
import shutil
import subprocess

import pytest

import sparse_attention_indexer_kpool_amd as kp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_consumer(tmp_path):
    kp.lib()                      # the library is built (fails loudly otherwise)
    pkg = os.path.dirname(os.path.abspath(kp.LIB_PATH))
    exe = tmp_path / "consumer"
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi", "consumer.c"),
           "-L", pkg, "-lkpool", f"-Wl,-rpath,{pkg}", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ)
    env["LD_LIBRARY_PATH"] = os.pathsep.join(
        [pkg, "/opt/rocm/lib", env.get("LD_LIBRARY_PATH", "")])
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
