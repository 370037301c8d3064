"""Plain CPU oracle of the k-nearest-neighbour distogram (pair-feature preprocessing).

TEST INFRASTRUCTURE ONLY.  This file is imported by tests/, by
__graft_entry__.smoke() and by the cpu_baseline leg of bench.py, and by
nothing else.  It shares no code with the HIP library and does not import it.

What it computes (FlashIPA rebuttal, paperhub page, answer to Q6): for each
residue only the distances to its k nearest neighbours are kept, as a
(B, L, k, n_bins) distogram instead of (B, L, L, n_bins), the neighbours
being found from the full L x L distance matrix of the residue positions.

The page leaves the arithmetic open; the readings taken here are:

  * positions are the frame translations t_i (fp32); the squared distance is
    formed in fp32 as ((dx*dx + dy*dy) + dz*dz) with d = t_j - t_i, every
    operation rounded to nearest (no fused multiply-add), and the distance is
    the correctly rounded fp32 square root.  fp32 is the precision of the
    coordinates, so the neighbour order and the bins are decided in it;
  * the candidates of residue i are the valid residues j != i of the same
    sample; they are ordered by squared distance, equal squared distances by
    the lower index first, and the first k are kept;
  * slots beyond the number of candidates hold index -1, distance +inf and an
    all-zero one-hot row; an invalid residue gets such a row in every slot;
  * the n_bins bins split [0, dmax) into equal widths w = fl32(dmax / n_bins);
    bin = floor(fl32(d / w)), and every d with fl32(d / w) >= n_bins goes to
    the last bin.

knn_distogram() is the vectorised form (one row block at a time, O(rows * L)
memory); knn_loops() is the same definition as pure-Python loops for tiny
inputs.  Both are pinned by tests/test_knn_oracle.py (hand-worked example,
closed form on a line, lattice ties, agreement with the float64 distance
order within the fp32 error bound, invariants of the selection, masks).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


def bin_width(dmax: float, nbins: int) -> np.float32:
    """Width of one distance bin, fl32(dmax / nbins)."""
    return np.float32(np.float32(dmax) / np.float32(nbins))


def sqdist_f32(ti: np.ndarray, tj: np.ndarray) -> np.ndarray:
    """fp32 squared distance ((dx*dx + dy*dy) + dz*dz), d = tj - ti, each op rounded.

    ti [..., 3] and tj [..., 3] broadcast against each other."""
    ti = np.asarray(ti, dtype=np.float32)
    tj = np.asarray(tj, dtype=np.float32)
    with np.errstate(over="ignore"):      # an overflow to +inf is a value like any other
        dx = tj[..., 0] - ti[..., 0]
        dy = tj[..., 1] - ti[..., 1]
        dz = tj[..., 2] - ti[..., 2]
        return (dx * dx + dy * dy) + dz * dz


def distance_bins(dist: np.ndarray, nbins: int, dmax: float) -> np.ndarray:
    """Bin of each fp32 distance: floor(fl32(d / w)), clamped to nbins-1 (an
    overflowed d = +inf of a real neighbour included)."""
    d = np.asarray(dist, dtype=np.float32)
    w = bin_width(dmax, nbins)
    with np.errstate(over="ignore", invalid="ignore"):
        q = d / w
    out = np.where(q >= np.float32(nbins), nbins - 1, np.floor(np.where(np.isfinite(q), q, 0.0)))
    return out.astype(np.int32)


def one_hot(bins: np.ndarray, nbins: int) -> np.ndarray:
    """[..., k] bins -> [..., k, nbins] fp32 one-hot; bin -1 gives an all-zero row."""
    out = np.zeros(bins.shape + (nbins,), dtype=np.float32)
    ii = np.nonzero(bins >= 0)
    out[ii + (bins[ii],)] = 1.0
    return out


def knn_distogram(translation: np.ndarray, mask: Optional[np.ndarray] = None, k: int = 20,
                  nbins: int = 20, dmax: float = 20.0, rows: Optional[Sequence[int]] = None,
                  block: int = 256) -> dict:
    """k nearest neighbours and their one-hot distogram for residues `rows`.

    translation [B,N,3] (cast to fp32), mask [B,N] bool or None (all valid).
    Returns index [B,R,k] int32, dist [B,R,k] fp32, bins [B,R,k] int32 and
    dgram [B,R,k,nbins] fp32 for R = len(rows) (all residues if None)."""
    t = np.asarray(translation, dtype=np.float32)
    B, N, _ = t.shape
    valid = np.ones((B, N), dtype=bool) if mask is None else np.asarray(mask, dtype=bool)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    R = len(rows)
    index = np.full((B, R, k), -1, dtype=np.int32)
    dist = np.full((B, R, k), np.inf, dtype=np.float32)
    for b in range(B):
        for r0 in range(0, R, block):
            rr = rows[r0:r0 + block]
            d2 = sqdist_f32(t[b, rr][:, None, :], t[b][None, :, :])       # [rb, N]
            for a, i in enumerate(rr):
                if not valid[b, i]:
                    continue
                cand = np.nonzero(valid[b] & (np.arange(N) != i))[0]     # ascending j
                order = cand[np.argsort(d2[a, cand], kind="stable")][:k]
                n = len(order)
                index[b, r0 + a, :n] = order
                dist[b, r0 + a, :n] = np.sqrt(d2[a, order])
    bins = np.where(index >= 0, distance_bins(dist, nbins, dmax), -1).astype(np.int32)
    return dict(index=index, dist=dist, bins=bins, dgram=one_hot(bins, nbins))


def knn_loops(translation, mask=None, k: int = 20, nbins: int = 20, dmax: float = 20.0) -> dict:
    """The same definition as pure-Python loops over fp32 scalars (tiny inputs only)."""
    t = np.asarray(translation, dtype=np.float32)
    B, N, _ = t.shape
    valid = np.ones((B, N), dtype=bool) if mask is None else np.asarray(mask, dtype=bool)
    w = bin_width(dmax, nbins)
    index = np.full((B, N, k), -1, dtype=np.int32)
    dist = np.full((B, N, k), np.inf, dtype=np.float32)
    bins = np.full((B, N, k), -1, dtype=np.int32)
    for b in range(B):
        for i in range(N):
            if not valid[b, i]:
                continue
            keyed = []
            for j in range(N):
                if j == i or not valid[b, j]:
                    continue
                with np.errstate(over="ignore"):
                    parts = [np.float32(t[b, j, c] - t[b, i, c]) for c in range(3)]
                    s = np.float32(np.float32(parts[0] * parts[0]) + np.float32(parts[1] * parts[1]))
                    s = np.float32(s + np.float32(parts[2] * parts[2]))
                keyed.append((s, j))
            keyed.sort()
            for slot, (s, j) in enumerate(keyed[:k]):
                d = np.float32(np.sqrt(s))
                q = np.float32(d / w)
                index[b, i, slot] = j
                dist[b, i, slot] = d
                bins[b, i, slot] = nbins - 1 if q >= nbins else int(np.floor(q))
    return dict(index=index, dist=dist, bins=bins, dgram=one_hot(bins, nbins))
