"""Host-only fuzz of the pool metadata in csrc/pool.cpp: random open / append / batched append /
fork / snapshot / fork-from-snapshot / release / close sequences on planning pools, checked
against an independent model after every call (ring tags, page holdings, window-safe length by
brute force, free pages, byte accounting, error codes).  Compiled with g++ and AddressSanitizer /
UBSan; the HIP runtime and the kernel launchers are stubs that abort if reached.  See
pool_fuzz_check.cpp."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "long_context_swa_amd", "csrc")
HIP_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(HIP_INCLUDE),
                    reason="needs g++ and the HIP headers")
def test_pool_metadata_matches_model_under_sanitizers(tmp_path):
    exe = str(tmp_path / "pool_fuzz")
    subprocess.run(["g++", "-std=c++20", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-I", HIP_INCLUDE,
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                    os.path.join(CSRC, "pool.cpp"), os.path.join(HERE, "pool_fuzz_check.cpp"), "-o", exe],
                   check=True, capture_output=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "pool_fuzz_mismatches=0" in r.stdout
