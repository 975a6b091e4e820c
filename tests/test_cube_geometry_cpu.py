"""The library's latent-grid cube helpers (csrc/common.hpp: cube_at, cube_token,
cube_len_of_flags), compiled for the host, list the same cubes and tokens as the
oracle's cube_tiles on ragged and whole grids."""
import os
import subprocess
import sys

import pytest

from oracle import vsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"


@pytest.fixture(scope="module")
def prog(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("cube") / "cube_geometry")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", f"-I{ROOT}/long_sequence_attention_amd/csrc",
                    f"-I{ROOT}/include", os.path.join(ROOT, "tests", "host", "cube_geometry.hip"), "-o", exe],
                   check=True, capture_output=True)
    return exe


@pytest.mark.parametrize("grid", [(5, 5, 4), (5, 6, 7), (21, 45, 80), (3, 5, 7), (8, 5, 8), (1, 1, 1), (8, 16, 16)])
def test_cube_helpers_match_oracle(prog, grid):
    out = subprocess.run([prog, *map(str, grid)], capture_output=True, text=True, check=True).stdout.split("\n")
    cubes = vsa.cube_tiles(grid)
    lines = [l for l in out if l.strip()]
    assert len(lines) == len(cubes)
    for line, c in zip(lines, cubes):
        vals = [int(x) for x in line.split()]
        assert vals[0] == len(c) and vals[1:] == c.tolist()
