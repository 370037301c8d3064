"""Pins of the kNN-distogram oracle against what the pages and plain mathematics fix.

The definition is the k-nearest-neighbour distogram of the FlashIPA rebuttal
(paperhub page, answer to Q6).  Each test targets a different part of it so
that a plausible slip -- a dropped coordinate, the query counted as its own
neighbour, ties taken in the wrong order, an off-by-one bin, a mask ignored,
the wrong row written -- fails at least one of them.
"""
import json
import os

import numpy as np
import pytest

from oracle import bin_width, distance_bins, knn_distogram, knn_loops, one_hot, sqdist_f32
from rna_structure_amd import synth
from rna_structure_amd.synth import IPAShape, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    with open(os.path.join(GOLDEN, "knn_worked_example.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("impl", ["vector", "loops"])
def test_hand_worked_example(impl):
    """Six integer points, three masks: neighbours, distances and bins worked by hand."""
    g = _golden()
    pts = np.array(g["points"], dtype=np.float32)
    for case in g["cases"]:
        mask = np.array(case["mask"], dtype=bool)[None]
        fn = knn_distogram if impl == "vector" else knn_loops
        out = fn(pts[None], mask, k=g["k"], nbins=g["nbins"], dmax=g["dmax"])
        assert np.array_equal(out["index"][0], np.array(case["index"])), case["mask"]
        assert np.array_equal(out["bins"][0], np.array(case["bins"])), case["mask"]
        sq = np.array(case["sqdist"], dtype=np.float64)
        want = np.where(sq < 0, np.inf, np.sqrt(np.maximum(sq, 0)))
        fin = np.isfinite(want)
        assert np.array_equal(np.isfinite(out["dist"][0]), fin)
        # the fp32 distance is the correctly rounded square root of an exact integer
        assert np.array_equal(out["dist"][0][fin], want[fin].astype(np.float32))
        oh = out["dgram"][0]
        assert np.array_equal(oh.sum(-1), fin.astype(np.float32))
        assert np.array_equal(np.argmax(oh, -1)[fin], np.array(case["bins"])[fin])


def test_points_on_a_line_closed_form():
    """x_i = 4i: the m-th ring of neighbours is {i-m, i+m} at distance 4m, lower index
    first, so the slots follow i-1, i+1, i-2, i+2, ... with one-sided runs at the ends."""
    N, k, nbins, dmax = 40, 7, 8, 16.0
    t = np.zeros((1, N, 3), dtype=np.float32)
    t[0, :, 0] = 4.0 * np.arange(N)
    out = knn_distogram(t, None, k=k, nbins=nbins, dmax=dmax)
    for i in range(N):
        want = []
        m = 1
        while len(want) < k:
            for j in (i - m, i + m):
                if 0 <= j < N and len(want) < k:
                    want.append((j, 4 * m))
            m += 1
        assert out["index"][0, i].tolist() == [j for j, _ in want], i
        assert out["dist"][0, i].tolist() == [float(d) for _, d in want], i
        # width 2: bin of distance 4m is 2m, clamped to the last bin
        assert out["bins"][0, i].tolist() == [min(2 * (d // 4), nbins - 1) for _, d in want], i


def test_lattice_ties_against_exact_integers():
    """A 4x4x3 unit lattice has many equal distances: the selection equals a brute-force
    sort of exact integer squared distances by (distance, index)."""
    g = np.stack(np.meshgrid(np.arange(4), np.arange(4), np.arange(3), indexing="ij"), -1).reshape(-1, 3)
    rng = np.random.default_rng(3)
    perm = rng.permutation(len(g))
    pts = g[perm]
    N, k = len(pts), 12
    mask = np.ones(N, dtype=bool)
    mask[[5, 17, 30]] = False
    out = knn_distogram(pts[None].astype(np.float32), mask[None], k=k, nbins=6, dmax=3.0)
    for i in range(N):
        if not mask[i]:
            assert np.all(out["index"][0, i] == -1)
            continue
        cand = [(int(((pts[j] - pts[i]) ** 2).sum()), j) for j in range(N) if j != i and mask[j]]
        cand.sort()
        assert out["index"][0, i].tolist() == [j for _, j in cand[:k]], i
        assert np.array_equal(out["dist"][0, i], np.sqrt(np.array([d for d, _ in cand[:k]], dtype=np.float64)).astype(np.float32))


@pytest.mark.parametrize("frames", ["walk", "gauss"])
def test_selection_agrees_with_float64_distances(frames):
    """Against distances recomputed in float64 from the same fp32 coordinates: every
    kept distance is within the fp32 error bound of the exact one, the kept slots are
    ordered, and no dropped candidate is nearer than a kept one beyond that bound.
    A dropped coordinate, a wrong operand or a missed candidate fails this."""
    s = IPAShape(B=2, N=300, H=1, dtype="f32")
    inp = make_inputs(s, 5, frames=frames, step=3.8, trans_sigma=10.0, lengths=(200, 300))
    t32 = inp["translation"].astype(np.float32)
    mask = inp["mask"]
    k = 20
    out = knn_distogram(t32, mask, k=k)
    t64 = t32.astype(np.float64)
    rel = 1e-6
    for b in range(2):
        D = np.sqrt(((t64[b][:, None] - t64[b][None]) ** 2).sum(-1))
        for i in range(300):
            idx = out["index"][b, i]
            if not mask[b, i]:
                assert np.all(idx == -1)
                continue
            kept = idx[idx >= 0]
            assert len(kept) == min(k, int(mask[b].sum()) - 1)
            assert np.all(mask[b, kept]) and i not in kept
            d = out["dist"][b, i][: len(kept)].astype(np.float64)
            assert np.all(np.abs(d - D[i, kept]) <= rel * D[i, kept] + 1e-30)
            assert np.all(np.diff(D[i, kept]) >= -rel * D[i, kept][1:])
            others = np.setdiff1d(np.nonzero(mask[b])[0], np.append(kept, i))
            if len(others):
                assert D[i, others].min() >= D[i, kept].max() * (1 - 2 * rel)


def test_loops_equal_vectorised_with_masks_and_ties():
    """The loop form and the vectorised form agree bit for bit, ties included."""
    rng = np.random.default_rng(7)
    t = rng.integers(-3, 4, size=(2, 23, 3)).astype(np.float32)   # many exact ties
    t[1] = rng.standard_normal((23, 3)).astype(np.float32) * 5
    mask = rng.random((2, 23)) > 0.2
    for k in (1, 5, 30):
        a = knn_distogram(t, mask, k=k, nbins=5, dmax=6.0)
        b = knn_loops(t, mask, k=k, nbins=5, dmax=6.0)
        for key in ("index", "dist", "bins", "dgram"):
            assert np.array_equal(a[key], b[key]), (k, key)


def test_rows_subset_and_row_blocks():
    """Selected rows equal the same rows of the full computation, for any row blocking."""
    s = IPAShape(B=1, N=700, H=1, dtype="f32")
    inp = make_inputs(s, 9, frames="walk", step=6.0)
    full = knn_distogram(inp["translation"], inp["mask"], k=20)
    rows = np.array([0, 1, 255, 256, 257, 511, 699])
    sub = knn_distogram(inp["translation"], inp["mask"], k=20, rows=rows, block=3)
    for key in ("index", "dist", "bins", "dgram"):
        assert np.array_equal(sub[key], full[key][:, rows]), key


def test_bins_at_edges():
    """floor(d / w) with w = dmax / nbins: exact edges go up, just below stays, d >= dmax
    and huge d (even an overflowed +inf) clamp to the last bin."""
    nb, dmax = 20, 20.0
    assert bin_width(dmax, nb) == np.float32(1.0)
    d = np.array([0.0, 0.5, 1.0, np.nextafter(np.float32(1.0), np.float32(0.0)), 19.0,
                  np.nextafter(np.float32(20.0), np.float32(0.0)), 20.0, 250.0, 3e38, np.inf],
                 dtype=np.float32)
    assert distance_bins(d, nb, dmax).tolist() == [0, 0, 1, 0, 19, 19, 19, 19, 19, 19]
    # a width that is not a power of two: bins of 3.0 are floor(fl32(d / fl32(0.6)))
    w = bin_width(6.0, 10)
    assert w == np.float32(0.6)
    d = np.array([0.6, 1.2, 1.8, 5.99, 6.0], dtype=np.float32)
    want = [int(np.floor(np.float32(x) / w)) for x in d]
    want = [min(v, 9) for v in want]
    assert distance_bins(d, 10, 6.0).tolist() == want
    oh = one_hot(np.array([[2, -1, 0]]), 3)
    assert oh.tolist() == [[[0, 0, 1], [0, 0, 0], [1, 0, 0]]]


def _exact_rn32(fr):
    """Round a rational to the nearest fp32 (ties to even), from exact comparisons."""
    from fractions import Fraction
    f = np.float32(float(fr))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    return min(cands, key=lambda c: (abs(Fraction(float(c)) - fr), int(c.view(np.uint32)) & 1))


def test_sqdist_rounding_order():
    """The squared distance is ((dx*dx + dy*dy) + dz*dz) in fp32, each op rounded.  For
    this difference vector the other summation order and the fused multiply-add chain
    fma(dz, dz, fma(dy, dy, dx*dx)) both give other bits; all three stay within the fp32
    error bound of the exact value."""
    from fractions import Fraction
    d = np.array([0x3F70ABE6, 0xC0EDEB75, 0xC11379DF], dtype=np.uint32).view(np.float32)
    got = sqdist_f32(np.zeros(3, dtype=np.float32), d)
    dx, dy, dz = d
    assert got == np.float32(np.float32(dx * dx + dy * dy) + np.float32(dz * dz))
    other = np.float32(dx * dx + np.float32(dy * dy + dz * dz))
    t = _exact_rn32(Fraction(float(dy)) ** 2 + Fraction(float(np.float32(dx * dx))))
    fused = _exact_rn32(Fraction(float(dz)) ** 2 + Fraction(float(t)))
    assert got != other and got != fused
    exact = sum(Fraction(float(c)) ** 2 for c in d)
    for v in (got, other, fused):
        assert abs(Fraction(float(v)) - exact) <= 3 * Fraction(2) ** -24 * exact


def test_matches_synthetic_distogram_recipe():
    """The one-hot channels that the synthetic inputs put into the first pair channels
    (bins of the (r+1)-th nearest residue, 20 bins on [0, 20)) are the first slots of
    the distogram, computed here independently in fp32.  The synthetic recipe works in
    float64, so the walk step is kept off the bin edges (with a 6 A step every chain
    neighbour sits on the 6 A edge, where float64 and fp32 round to different sides)."""
    s = IPAShape(B=2, N=400, H=1, R=2, dtype="f32")
    inp = make_inputs(s, 12, frames="walk", step=3.8)
    ref = synth._distogram_channels(inp["translation"], 2, nbins=20)
    out = knn_distogram(inp["translation"], None, k=2, nbins=20, dmax=20.0)
    assert np.array_equal(out["dgram"], ref.astype(np.float32))


def test_empty_and_tiny():
    """N=1 or a single valid residue: no candidates at all; k larger than N-1."""
    t = np.zeros((1, 1, 3), dtype=np.float32)
    out = knn_distogram(t, None, k=4)
    assert np.all(out["index"] == -1) and np.all(np.isinf(out["dist"])) and not out["dgram"].any()
    t = np.array([[[0, 0, 0], [1, 0, 0], [0, 2, 0]]], dtype=np.float32)
    out = knn_distogram(t, None, k=5, nbins=4, dmax=4.0)
    assert out["index"][0].tolist() == [[1, 2, -1, -1, -1], [0, 2, -1, -1, -1], [0, 1, -1, -1, -1]]
    assert out["bins"][0, 1].tolist() == [1, 2, -1, -1, -1]
    # a real neighbour whose squared distance overflows fp32 keeps its index, has
    # distance +inf and falls in the last bin
    t = np.array([[[0, 0, 0], [3e19, 0, 0]]], dtype=np.float32)
    for fn in (knn_distogram, knn_loops):
        out = fn(t, None, k=2, nbins=4, dmax=4.0)
        assert out["index"][0].tolist() == [[1, -1], [0, -1]]
        assert np.all(np.isinf(out["dist"][0]))
        assert out["bins"][0].tolist() == [[3, -1], [3, -1]]
