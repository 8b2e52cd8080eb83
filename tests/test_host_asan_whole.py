"""Host side of the whole-T cache under AddressSanitizer and UBSan (CPU, no GPU).

kvqw_api.cpp is compiled with g++ together with CPU stand-ins for the HIP calls it makes and for the
three kernel launches (tests/host_asan/whole_host_stubs.cpp).  Each stand-in checks that every pointer
the launch would hand a kernel, with the extent that kernel touches (codes, metadata, inputs, the split
and tile workspace, q, out), lies inside the buffers the caller allocated.  The driver replays the two
whole-T workloads the bench runs.  A host SIGSEGV was once recorded inside the HIP launch path of
kvqw_decode_attn under a hardware-counter profiler; this test shows the library's host code hands that
launch only in-bounds arguments."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"), reason="needs g++ and HIP headers")
def test_whole_t_host_path_is_memory_clean(tmp_path):
    exe = str(tmp_path / "whole_host")
    csrc = os.path.join(ROOT, "quantized_kv_cache_kivi_amd", "csrc")
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + csrc, "-o", exe,
           os.path.join(ROOT, "tests", "host_asan", "whole_host_stubs.cpp"), os.path.join(csrc, "kvqw_api.cpp")]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-3000:]
    assert "no host memory error" in r.stdout
