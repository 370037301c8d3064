"""GPU check of ipa_forward_noalloc (the forward that allocates nothing, its
buffers in a static device array) against the three-call forward
(ipa_lift, ipa_flash_fwd, ipa_epilogue) on the same inputs: two calls in a
row, the second with a smaller input, so that whatever the first call left in
the shared array cannot pass for the second's results.  The same kernels run
in the same launch configurations, so the outputs are compared bit for bit
(and against the oracle within the bf16 bar)."""
import types

import numpy as np
import pytest

from oracle import ipa_factored
from rna_structure_amd.synth import IPAShape, make_inputs

from gpu_helpers import add_guards, check_guards, max_abs_rel, run_gpu, say

pytestmark = pytest.mark.gpu


def _noalloc(inp):
    import torch
    from rna_structure_amd import _lib
    shape = inp["shape"]
    t = _lib.device_inputs(inp, "cuda")
    s = _lib.make_shape(shape, inp["eps"])
    # outputs NaN-poisoned between guard bands of sentinel bytes
    bufs = types.SimpleNamespace(
        update=torch.full((shape.B, shape.N, shape.Cout), float("nan"), dtype=torch.float32, device="cuda"),
        local=torch.full((shape.B, shape.N, shape.H, shape.Q, 3), float("nan"), dtype=torch.float32, device="cuda"))
    add_guards(bufs, ("update", "local"))
    bufs.update.fill_(float("nan"))
    bufs.local.fill_(float("nan"))
    update, local = bufs.update, bufs.local
    _lib.ipa_forward_noalloc(s, t, update, local)
    torch.cuda.synchronize()
    check_guards(bufs)
    return update.cpu().numpy().astype(np.float64), local.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("first,second", [
    # protein-like batch (B8 N256 H8, ragged, pair-mask dropout, an empty row), then a smaller one
    ((IPAShape(B=8, N=256, H=8), 71, dict(frames="walk", step=3.8, lengths=(128, 256), pair_dropout=0.05,
                                             empty_row=True)),
     (IPAShape(B=2, N=100, H=8), 72, dict(frames="walk", step=3.8, lengths=(60, 100)))),
    # RNA-like length (B1 N2048 H8, no pair mask), then a smaller fp32 problem
    ((IPAShape(B=1, N=2048, H=8), 73, dict(frames="walk", step=6.0)),
     (IPAShape(B=1, N=16, H=4, Cz=16, dtype="f32"), 74, dict(frames="gauss", trans_sigma=10.0, masked_keys=(5,)))),
])
def test_noalloc_forward_matches_three_calls(first, second):
    for shape, seed, kw in (first, second):
        say(f"case noalloc {shape} seed={seed}")
        inp = make_inputs(shape, seed, **kw)
        upd, loc = _noalloc(inp)
        _, _, ref = run_gpu(inp)
        assert np.array_equal(upd, ref["update"]), "update differs from the three-call forward"
        assert np.array_equal(loc, ref["local_points"]), "local_points differ from the three-call forward"
        tol = 1e-4 if shape.dtype == "f32" else 2e-2
        rows = np.arange(min(shape.N, 64))
        orc = ipa_factored(inp, rows=rows, keep=("update", "local_points"))
        e1 = max_abs_rel(upd[:, rows], orc["update"])
        e2 = max_abs_rel(loc[:, rows], orc["local_points"])
        say(f"  bit-identical to the three calls; oracle rows 0..{rows[-1]}: update {e1:.2e} local_points {e2:.2e}")
        assert e1 <= tol and e2 <= tol
