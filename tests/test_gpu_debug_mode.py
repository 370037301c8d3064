"""FLASHIPA_DEBUG: with the variable set, every call waits for its kernels
(and would name a failing one on stderr); the results are those of the
ordinary calls.  The variable is read once per process, so the debug run is a
child process."""
import os
import subprocess
import sys

import numpy as np
import pytest

from rna_structure_amd.synth import IPAShape, make_inputs

from gpu_helpers import run_gpu, say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys, numpy as np
sys.path.insert(0, sys.argv[1]); sys.path.insert(0, sys.argv[1] + "/tests")
from rna_structure_amd.synth import IPAShape, make_inputs
from gpu_helpers import run_gpu
inp = make_inputs(IPAShape(B=2, N=150, H=4), 61, frames="walk", step=3.8, lengths=(90, 150), pair_dropout=0.05)
_, _, out = run_gpu(inp)
np.save(sys.argv[2], out["update"])
np.save(sys.argv[3], out["local_points"])
"""


def test_debug_mode_gives_the_same_results(tmp_path):
    say("case FLASHIPA_DEBUG=1 in a child process")
    upd, loc = str(tmp_path / "u.npy"), str(tmp_path / "l.npy")
    env = dict(os.environ, FLASHIPA_DEBUG="1")
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT, upd, loc], env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "flashipa:" not in r.stderr
    inp = make_inputs(IPAShape(B=2, N=150, H=4), 61, frames="walk", step=3.8, lengths=(90, 150), pair_dropout=0.05)
    _, _, out = run_gpu(inp)
    assert np.array_equal(np.load(upd), out["update"])
    assert np.array_equal(np.load(loc), out["local_points"])
