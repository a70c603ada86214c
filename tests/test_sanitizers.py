"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The CPU oracle (oracle/mx_oracle.c) and the C-ABI validation layer
(microscaling_block_scaled_amd/csrc/mx_api.cpp, with its kernel launchers
replaced by recording stubs) are built with gcc / g++ and
-fsanitize=address,undefined -fno-sanitize-recover=all, and driven through
every entry point on whole and ragged shapes; any report fails the test.
No GPU code is involved."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g",
       "-O1"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, (" ".join(cmd), r.stdout[-2000:], r.stderr[-4000:])
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11", *SAN, "-fopenmp", "-ffp-contract=off", "-I" + os.path.join(ROOT, "oracle"),
          os.path.join(HERE, "helpers", "oracle_sanitize_main.c"), os.path.join(ROOT, "oracle", "mx_oracle.c"),
          "-lm", "-o", exe])
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1")
    r = _run([exe], env=env)
    assert "ran clean" in r.stdout


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the HIP headers not available")
def test_api_validation_under_sanitizers(tmp_path):
    exe = str(tmp_path / "api_san")
    csrc = os.path.join(ROOT, "microscaling_block_scaled_amd", "csrc")
    _run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
          "-I" + os.path.join(ROOT, "include"), "-I" + csrc,
          os.path.join(HERE, "helpers", "api_sanitize_main.cpp"), os.path.join(csrc, "mx_api.cpp"),
          "-o", exe])
    r = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert "all checks passed" in r.stdout
