"""The kernels' grid-stride loops: with ZERO_BLOCKS_PER_CU the launches use a
grid capped at that many workgroups per compute unit, so every workgroup
processes several tiles, the last one ragged (the form that arrays beyond
the uncapped grid of 2^24 tiles take).  The setting is read once per process,
so each case runs tests/grid_capped_child.py in a child process, which checks
every streaming kernel against the oracle."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("blocks_per_cu", ["1", "3"])
def test_grid_capped_kernels_match_oracle(blocks_per_cu):
    print(f"grid-capped child: ZERO_BLOCKS_PER_CU={blocks_per_cu}", flush=True)
    env = dict(os.environ, ZERO_BLOCKS_PER_CU=blocks_per_cu)
    r = subprocess.run([sys.executable, os.path.join(HERE, "grid_capped_child.py")], env=env,
                       capture_output=True, text=True, timeout=300)
    print(r.stdout[-3000:], flush=True)
    assert r.returncode == 0, r.stderr[-3000:]
    assert "all kernels match the oracle" in r.stdout
