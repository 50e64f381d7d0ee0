"""The C-ABI layer's host code under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU: api.cpp is compiled with both
sanitizers on its host side (the device side of the kernels is untouched),
linked with the library's other objects into tests/sanitize/abi_driver.cpp,
and run; every call fails validation, so no kernel is launched. Runs only
where no GPU is visible."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sparse_attention_indexer_kpool_amd")


def _no_gpu_visible():
    import torch
    return torch.cuda.device_count() == 0


@pytest.mark.skipif(not _no_gpu_visible(), reason="host-only sanitizer run, no GPU wanted")
@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    from sparse_attention_indexer_kpool_amd import build as b
    objs = []
    for src in b.SOURCES:
        if src == "api.cpp":
            continue
        o = os.path.join(b.BUILD, os.path.splitext(src)[0] + ".o")
        if not os.path.exists(o):
            b.build(verbose=False)
        objs.append(o)
    api_o = str(tmp_path / "api_san.o")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    cmd = [b.hipcc(), *b.FLAGS, "-O1", "-g", *san, "-c", os.path.join(b.CSRC, "api.cpp"),
           "-o", api_o]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    drv_o = str(tmp_path / "driver.o")
    r = subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=undefined", f"-I{ROOT}/include", "-c",
                        os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"), "-o", drv_o],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    exe = str(tmp_path / "abi_driver")
    r = subprocess.run(["g++", "-fsanitize=address,undefined", drv_o, api_o, *objs,
                        "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64",
                        "-lrocprofiler-sdk-roctx", "-pthread", "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all sanitized checks passed" in r.stdout
