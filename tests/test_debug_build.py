"""Debug and sanitizer builds of the library's host code (CPU only).

The C-ABI source is compiled with TREE_ATTN_DEBUG (which adds the host-side
checker tree_attn_debug_check_verify) and AddressSanitizer on the host
side, linked with tests/abi_sanitize.cpp, and run: argument checks of the
launch entry points, planning over a sweep of shapes, and the debug
checker naming planted out-of-range values.  Any ASan report or failed
expectation fails the test."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tree_masked_attention_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
# sanitizer flags apply to the host compilation only
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.fixture(scope="module")
def asan_driver(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("asan") / "abi_sanitize")
    cmd = ([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
            "-DTREE_ATTN_DEBUG", "-Xclang", "-target-feature", "-Xclang",
            "-packed-fp32-ops"] + HOST_ASAN +
           ["-I", os.path.join(ROOT, "include"), "-I", CSRC,
            os.path.join(CSRC, "tree_attn.hip"),
            os.path.join(ROOT, "tests", "abi_sanitize.cpp"), "-o", out])
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-4000:]
    return out


def test_host_code_under_asan(asan_driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               HIP_VISIBLE_DEVICES="")
    res = subprocess.run([asan_driver], capture_output=True, text=True,
                         timeout=300, env=env)
    print(res.stdout[-4000:])
    assert "AddressSanitizer" not in res.stderr, res.stderr[-4000:]
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-2000:]
    assert res.stdout.strip().endswith("ok: 0 failure(s)")
