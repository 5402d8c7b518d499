"""Every GEMM tile configuration against the oracle. The library reads its
tile override (SQ_GEMM_TILE: 0 generic, 1 256x256, 2 128x128, 3 256x192,
4 skinny and 5 decode, which apply where M <= 64; 5 only without LoRA, the
other shapes then take the default rule) once per process, so each configuration runs gemm_tile_check.py in a child
process; the shapes there are ragged against every tile size and cover the
pipelined kernel's one-, two- and three-K-tile paths."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("tile", [0, 1, 2, 3, 4, 5])
def test_gemm_tile_config(tile):
    env = dict(os.environ, SQ_GEMM_TILE=str(tile))
    r = subprocess.run([sys.executable, os.path.join(HERE, "gemm_tile_check.py")], env=env,
                       capture_output=True, text=True, timeout=300)
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert lines, f"no result (rc {r.returncode}):\n{r.stdout[-2000:]}\n{r.stderr[-2000:]}"
    res = json.loads(lines[-1])
    assert res["tile"] == str(tile)
    assert r.returncode == 0 and not res["failures"], res
    assert res["cases"] == 9 * 9
