"""Host-only regression test of the pinned staging ring's reuse rule (csrc/staging_ring.h):
compiled with g++ (AddressSanitizer/UBSan on) and run on the CPU.  See staging_ring_check.cpp."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "long_context_swa_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_staging_ring_never_reuses_bytes_still_being_copied(tmp_path):
    exe = str(tmp_path / "ring_check")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-I", CSRC,
                    os.path.join(HERE, "staging_ring_check.cpp"), "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ring_space_violations=0" in r.stdout
