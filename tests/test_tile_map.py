"""The workgroup -> tile maps of the kernels (XCD remap, grouped raster,
split-K ranges) are bijections: built for the host from the kernels' own
header and checked over 5000 grid sizes and a sweep of tile grids, split
counts and raster group heights (CPU only)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_tile_maps_are_bijections(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = tmp_path / "tile_map_check"
    subprocess.run([hipcc, "--offload-host-only", "-x", "hip", "-O2", "-std=c++17",
                    os.path.join(HERE, "native", "tile_map_check.cpp"), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok ")
