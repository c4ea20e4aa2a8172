"""Host check of the attention kernel's LDS index maps (no GPU): the swizzles, the LDS
DMA source offsets and the per-lane operand read offsets of sage_tiles.h, compiled
into a host program (tests/host/index_maps_check.hip) that simulates one tile's copies
and reads for d = 64 and 128."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "host", "index_maps_check.hip")


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    pytest.skip("hipcc is needed to compile the host check")


def test_index_maps_stay_in_bounds_and_match_the_operand_layouts(tmp_path):
    exe = str(tmp_path / "index_maps_check")
    cmd = [_hipcc(), "-O1", "-std=c++20", "--offload-arch=gfx950", SRC, "-o", exe]
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert p.returncode == 0, p.stdout
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout
