"""GPU parity: the HIP path against the float64 CPU oracle on the same seeded
inputs.  Tolerance (max |gpu - ref| / max |ref| per output tensor): 1e-4 for
the fp32 path, 2e-2 for the bf16 matrix-core path; attention rows sum to
1 +- 1e-5."""
import math

import numpy as np
import pytest

from oracle import ipa_factored
from rna_structure_amd.synth import IPAShape, make_config, make_inputs

from gpu_helpers import add_guards, check_guards, compare, run_gpu, say

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _case(name, shape, seed, **kw):
    return pytest.param(shape, seed, kw, id=name)


SMALL = [
    _case("tiny-f32", IPAShape(B=1, N=16, H=4, Cz=16, dtype="f32"), 1016,
          frames="gauss", trans_sigma=10.0, masked_keys=(5,)),
    _case("ragged-bf16", IPAShape(B=2, N=200, H=4), 7, frames="walk", step=3.8, lengths=(100, 200),
          pair_dropout=0.1, empty_row=True),
    _case("ragged-f32", IPAShape(B=2, N=200, H=4, dtype="f32"), 8, frames="walk", step=3.8, lengths=(100, 200),
          pair_dropout=0.1, empty_row=True),
    _case("one-residue-bf16", IPAShape(B=3, N=1, H=2), 9, frames="gauss"),
    _case("one-residue-f32", IPAShape(B=3, N=1, H=2, dtype="f32"), 9, frames="gauss"),
    _case("n64-bf16", IPAShape(B=1, N=64, H=3), 10, frames="walk", step=3.8),
    _case("n65-bf16", IPAShape(B=1, N=65, H=3), 11, frames="walk", step=3.8, masked_keys=(64,)),
    _case("n129-f32", IPAShape(B=2, N=129, H=2, dtype="f32"), 12, frames="gauss", trans_sigma=20.0),
    _case("small-dims-bf16", IPAShape(B=2, N=70, H=3, D=4, Dv=3, P=2, Q=2, Cz=5, R=2, Cout=6), 13, frames="gauss"),
    _case("small-dims-f32", IPAShape(B=2, N=70, H=3, D=4, Dv=3, P=2, Q=2, Cz=5, R=2, Cout=6, dtype="f32"), 13,
          frames="gauss"),
    _case("mid-instance-bf16", IPAShape(B=1, N=150, H=2, D=16, Dv=16, P=4, Q=8, Cz=32, R=2), 14, frames="walk"),
    _case("rank1-p5-q9-bf16", IPAShape(B=1, N=100, H=2, D=8, Dv=8, P=5, Q=9, Cz=48, R=1, Cout=64), 15,
          frames="walk"),
    # one point per head up to three: every geometric-column layout of the lift
    _case("p1-q1-bf16", IPAShape(B=1, N=130, H=2, D=8, Dv=8, P=1, Q=1, Cz=16, R=1, Cout=32), 16, frames="walk",
          pair_dropout=0.1),
    _case("p2-q3-bf16", IPAShape(B=2, N=96, H=3, D=16, Dv=8, P=2, Q=3, Cz=24, R=2, Cout=48), 17, frames="walk",
          lengths=(50, 96)),
    _case("p3-q4-bf16", IPAShape(B=1, N=192, H=2, D=8, Dv=16, P=3, Q=4, Cz=40, R=2, Cout=64), 18, frames="gauss",
          trans_sigma=15.0, pair_dropout=0.05),
    # grids too small for the GPU: keys split into 4 and 2 ranges per query
    # tile, partial results merged by the combine kernel
    _case("split4-bf16", IPAShape(B=1, N=1024, H=2), 19, frames="walk", step=3.8, masked_keys=(5, 300, 1023)),
    _case("split2-ragged-bf16", IPAShape(B=2, N=600, H=3), 20, frames="walk", step=3.8, lengths=(300, 600),
          pair_dropout=0.05, empty_row=True),
    # rank-3 pair factors: the widest matrix-core instance (13 query K-steps,
    # 7 value blocks), once whole and once split into key ranges
    _case("rank3-bf16", IPAShape(B=2, N=300, H=3, R=3), 22, frames="walk", step=3.8, lengths=(200, 300),
          pair_dropout=0.05, empty_row=True),
    _case("rank3-split-bf16", IPAShape(B=1, N=1100, H=2, R=3), 23, frames="walk", step=3.8),
    # rank 1 at the standard widths (the per-head epilogue's rank-1 instance)
    _case("rank1-std-bf16", IPAShape(B=2, N=260, H=8, R=1), 24, frames="walk", step=3.8, lengths=(150, 260),
          pair_dropout=0.05, empty_row=True),
]


@pytest.mark.parametrize("shape,seed,kw", SMALL)
def test_parity_small(shape, seed, kw):
    say(f"case {shape} seed={seed}")
    inp = make_inputs(shape, seed, **kw)
    _, _, gpu = run_gpu(inp)
    compare(inp, gpu, tol=TOL[shape.dtype])


def test_all_masked_batch_is_zero():
    s = IPAShape(B=2, N=90, H=2)
    inp = make_inputs(s, 21, frames="walk")
    inp["mask"][1, :] = False
    say("case all-masked sample")
    _, _, gpu = run_gpu(inp)
    assert np.all(gpu["update"][1] == 0) and np.all(gpu["local_points"][1] == 0)
    assert np.all(np.isneginf(gpu["lse"][1]))
    compare(inp, gpu, tol=TOL["bf16"])


def _sample_rows(N, k, seed, extra=()):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(N, size=min(k, N), replace=False).tolist()) | {0, N - 1} | set(extra)
    return np.array(sorted(r for r in rows if 0 <= r < N))


@pytest.mark.parametrize("name", ["tiny", "protein"])
def test_parity_configs_full(name):
    inp = make_config(name)
    say(f"config {name} {inp['shape']}")
    _, _, gpu = run_gpu(inp)
    compare(inp, gpu, tol=TOL[inp["shape"].dtype])


def test_parity_rna_sampled():
    inp = make_config("rna")
    say(f"config rna {inp['shape']}")
    _, _, gpu = run_gpu(inp)
    compare(inp, gpu, rows=_sample_rows(2048, 48, 1), tol=TOL["bf16"])


def test_parity_short_batch_sampled():
    inp = make_config("short_batch")
    L0 = int(inp["mask"][0].sum())
    say(f"config short_batch {inp['shape']} empty row {L0 // 2}")
    _, _, gpu = run_gpu(inp)
    compare(inp, gpu, rows=_sample_rows(512, 24, 2, extra=(L0 // 2, L0 - 1, L0)), tol=TOL["bf16"])


@pytest.mark.parametrize("n", [4096, 8192, 16384, 32768])
def test_parity_sweep_sampled(n):
    inp = make_config(f"sweep_{n}")
    say(f"config sweep N={n}")
    _, _, gpu = run_gpu(inp)
    compare(inp, gpu, rows=_sample_rows(n, 6, 3, extra=(n // 2, n - 64, 63, 64)), tol=TOL["bf16"])


@pytest.mark.parametrize("R", [1, 3])
def test_parity_rank_sweep_sampled(R):
    """The rank sweep's shapes (B1 N8192 H8, pair factors of rank 1 and 3) at
    full size, on sampled rows."""
    inp = make_inputs(IPAShape(B=1, N=8192, H=8, R=R), 8100 + R, frames="walk", step=3.8)
    say(f"case rank sweep R={R} N=8192")
    _, _, gpu = run_gpu(inp)
    compare(inp, gpu, rows=_sample_rows(8192, 6, 4, extra=(63, 64, 4096, 8191)), tol=TOL["bf16"])


def _far_cluster_inputs(dtype):
    """B1 N192 H4: keys 128..191 (the third key tile) moved 180 A away along
    x; query row 10 may attend to those keys only (pair mask); the point
    weights 60, -60, 30, 0.5 (softplus of large arguments of both signs).  On
    the head with weight 60 every permitted logit of row 10 lies between
    -9.4e5 and -6.4e5 in log2 units: the page's softmax still normalises over
    those keys, and the row is not an empty neighbourhood."""
    from rna_structure_amd.synth import round_to
    s = IPAShape(B=1, N=192, H=4, dtype=dtype)
    inp = make_inputs(s, 41, frames="walk", step=3.8)
    tr = inp["translation"].astype(np.float64).copy()
    tr[0, 128:, 0] += 180.0
    inp["translation"] = round_to(tr, dtype)
    inp["point_weight_raw"] = round_to(np.array([60.0, -60.0, 30.0, 0.5]), dtype)
    pm = np.ones((1, 192, 192), dtype=bool)
    pm[0, 10, :128] = False
    inp["pair_mask"] = pm
    return inp


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_far_keys_and_extreme_point_weights(dtype):
    inp = _far_cluster_inputs(dtype)
    ref = ipa_factored(inp, rows=np.array([10]), keep=("logits", "lse", "empty"))
    permitted = ref["logits"][0, 0, 0, 128:] / math.log(2)
    assert permitted.max() < -5e5 and not ref["empty"][0, 0]
    say(f"case far keys {dtype}")
    _, _, gpu = run_gpu(inp)
    assert np.all(np.isfinite(gpu["lse"][0, :, 10]))
    compare(inp, gpu, rows=np.array([0, 5, 10, 11, 127, 128, 150, 191]), tol=TOL[dtype])


def test_chain_far_from_origin_bf16():
    """Every translation moved by (2e4, -1.5e4, 3e4) A before the bf16 rounding
    (spacing 128 A there): the centroids and centred points stay small."""
    from rna_structure_amd.synth import round_to
    s = IPAShape(B=2, N=300, H=4)
    inp = make_inputs(s, 43, frames="walk", step=3.8, lengths=(200, 300))
    tr = inp["translation"].astype(np.float64) + np.array([2e4, -1.5e4, 3e4])
    inp["translation"] = round_to(tr, "bf16")
    say("case chain far from the origin")
    _, _, gpu = run_gpu(inp)
    compare(inp, gpu, tol=TOL["bf16"])


@pytest.mark.parametrize("dtype,N", [("bf16", 300), ("f32", 300), ("bf16", 1100)])
def test_attention_rows_sum_to_one(dtype, N):
    """Attention rows a_ij = exp(L_ij - lse_i), from the logits the kernel uses and
    the kernel's log-sum-exp: they match the oracle's attention and sum to 1
    (N = 1100: log-sum-exp merged from 4 key ranges)."""
    import torch
    s = IPAShape(B=2, N=N, H=3, dtype=dtype)
    inp = make_inputs(s, 31, frames="walk", step=3.8, lengths=(2 * N // 3, N), pair_dropout=0.05, empty_row=True)
    say(f"case attention rows {dtype} N={N}")
    f, _, gpu = run_gpu(inp)
    rows = np.array([0, 7, 63, 64, 150, 199])
    ref = ipa_factored(inp, rows=rows, keep=("attention", "logits", "lse", "empty"))
    tol = TOL[dtype]
    for b in range(2):
        for h in range(3):
            L = f.logit_rows(b, h, int(rows[0]), int(rows[-1] - rows[0] + 1)).cpu().numpy().astype(np.float64)
            L = L[rows - rows[0]]
            lse = gpu["lse"][b, h, rows]
            for k, i in enumerate(rows):
                if ref["empty"][b, k]:
                    assert np.isneginf(lse[k]) and np.all(np.isneginf(L[k]))
                    continue
                a = np.exp(L[k] - lse[k])
                assert abs(a.sum() - 1.0) <= 1e-5, (b, h, i, a.sum())
                ra = ref["attention"][b, h, k]
                assert np.max(np.abs(a - ra)) <= tol * max(np.max(ra), 1e-30) + 1e-7, (b, h, i)
                perm = np.isfinite(L[k])
                lr = ref["logits"][b, h, k][perm]
                assert np.max(np.abs(L[k][perm] - lr)) <= (5e-2 if dtype == "bf16" else 1e-4) * max(1.0, np.abs(lr).max())


def test_deterministic():
    inp = make_config("protein")
    say("case determinism")
    _, _, g1 = run_gpu(inp)
    _, _, g2 = run_gpu(inp)  # run_gpu poisons the buffers again before the second forward
    for k in ("update", "local_points", "o", "lse"):
        assert not np.any(np.isnan(g1[k])), k
        assert np.array_equal(g1[k], g2[k]), k


@pytest.mark.parametrize("shape", [IPAShape(B=2, N=300, H=8), IPAShape(B=1, N=1024, H=2), IPAShape(B=1, N=100, H=2, dtype="f32")],
                         ids=["one-buffer", "split-keys", "f32"])
def test_repeated_calls_on_one_lift(shape):
    """ipa_flash_fwd and ipa_epilogue are functions of the lifted buffer and
    the inputs: called again on the same lift (outputs poisoned in between)
    they give the same bits, also where the keys are split over workgroups
    and merged."""
    import torch
    from rna_structure_amd import _lib
    inp = make_inputs(shape, 77, frames="walk", step=3.8, pair_dropout=0.05)
    say(f"case repeated calls {shape}")
    t = _lib.device_inputs(inp, "cuda")
    f = add_guards(_lib.FlashIPA(shape, eps=inp["eps"], with_pair_mask=True))
    f.poison()
    f.lift(t)
    outs = []
    for _ in range(3):
        for buf in (f.o, f.lse, f.update, f.local_points):
            buf.fill_(float("nan"))
        f.attend()
        f.epilogue(t)
        torch.cuda.synchronize()
        outs.append({k: v.detach().cpu().numpy().copy() for k, v in
                     dict(o=f.o, lse=f.lse, update=f.update, local_points=f.local_points).items()})
    for k in outs[0]:
        assert not np.any(np.isnan(outs[0][k])), k
        for o in outs[1:]:
            assert np.array_equal(outs[0][k], o[k]), k
    check_guards(f)


def test_rigid_invariance_gpu_f32():
    s = IPAShape(B=1, N=150, H=4, dtype="f32")
    inp = make_inputs(s, 41, frames="walk", step=3.8)
    say("case invariance f32")
    _, _, g1 = run_gpu(inp)
    rng = np.random.default_rng(5)
    qt = rng.standard_normal(4)
    qt /= np.linalg.norm(qt)
    w, x, y, z = qt
    G = np.array([[1 - 2 * (y * y + z * z), 2 * (x * y - z * w), 2 * (x * z + y * w)],
                  [2 * (x * y + z * w), 1 - 2 * (x * x + z * z), 2 * (y * z - x * w)],
                  [2 * (x * z - y * w), 2 * (y * z + x * w), 1 - 2 * (x * x + y * y)]])
    moved = dict(inp)
    moved["rotation"] = np.einsum("xy,bnyz->bnxz", G, inp["rotation"]).astype(np.float32).astype(np.float64)
    moved["translation"] = (np.einsum("xy,bny->bnx", G, inp["translation"]) + 100.0).astype(np.float32).astype(np.float64)
    _, _, g2 = run_gpu(moved)
    for k in ("update", "local_points"):
        assert np.all(np.isfinite(g1[k])) and np.all(np.isfinite(g2[k])), k
        err = np.max(np.abs(g1[k] - g2[k])) / np.max(np.abs(g1[k]))
        assert err <= 1e-4, (k, err)
