"""The tile-range helpers of the kernels' mask header against the element-wise mask rule, compiled
for the host with g++ (see tests/mask_tiles_check.cpp).  The relay route's turn numbering relies on
the key tiles that see a q tile being contiguous and starting at first_kv_tile."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_tile_ranges_match_element_mask(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "mask_tiles_check")
    res = subprocess.run([gxx, "-std=c++17", "-O2", "-I/opt/rocm/include", "-D__HIP_PLATFORM_AMD__",
                          os.path.join(HERE, "mask_tiles_check.cpp"), "-o", exe],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    out = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0 and out.stdout.startswith("ok"), out.stdout + out.stderr
