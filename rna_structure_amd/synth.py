"""Seeded synthetic inputs for the IPA forward, shared by the oracle tests, the
GPU parity tests and the benchmark.

This module only draws and rounds random numbers; it holds none of the
attention arithmetic (no logits, softmax, aggregation or projection), so that
neither the CPU oracle nor the HIP path depends on the other through it.

Argument names and layouts follow the problem statement of the "Invariant
point attention (IPA)" page (biotorch, "Required behavior"):
  q, k [B,N,H,D]; v [B,N,H,Dv]; q_points, k_points [B,N,H,P,3];
  v_points [B,N,H,Q,3]; rotation [B,N,3,3] (column-vector convention,
  x_global = R @ x + t); translation [B,N,3]; point_weight_raw [H];
  mask [B,N] (True = valid); pair_mask [B,N,N] (None = all valid);
  w_out [F,Cout] with F = H*(Dv+4Q+Cz); b_out [Cout].
The pair representation is given as rank-R factors zl, zr [B,N,R,Cz] with
per-head pair-bias weights w_pair [H,Cz] (the factorisation of the FlashIPA
rebuttal, paperhub page, answers to Q4/Q5).

Every floating array is generated in float64, rounded once to the run dtype
and returned as float64 holding exactly the rounded values, so every consumer
sees identical numbers.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = ["IPAShape", "make_inputs", "make_config", "CONFIGS", "round_to", "sweep_shapes"]


@dataclasses.dataclass(frozen=True)
class IPAShape:
    B: int
    N: int
    H: int
    D: int = 16
    Dv: int = 16
    P: int = 4
    Q: int = 8
    Cz: int = 64
    R: int = 2
    Cout: int = 128
    dtype: str = "bf16"  # "f32" or "bf16"

    @property
    def F(self) -> int:
        return self.H * (self.Dv + 4 * self.Q + self.Cz)

    @property
    def d_qk(self) -> int:
        # scalar + 3P point cross terms + 2 norm/constant columns + pair factor
        return self.D + 3 * self.P + 2 + self.R * self.Cz

    @property
    def d_v(self) -> int:
        return self.Dv + 3 * self.Q + self.R * self.Cz


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values once to the run dtype (round-to-nearest-even) and
    return them as float64."""
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)
    if dtype == "f32":
        return f.astype(np.float64)
    if dtype != "bf16":
        raise ValueError(dtype)
    u = f.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _quat_rotations(rng: np.random.Generator, n: int) -> np.ndarray:
    """Proper rotations from normalised N(0, I4) quaternions."""
    qt = rng.standard_normal((n, 4))
    qt /= np.linalg.norm(qt, axis=-1, keepdims=True)
    w, x, y, z = qt.T
    R = np.empty((n, 3, 3))
    R[:, 0, 0] = 1 - 2 * (y * y + z * z)
    R[:, 0, 1] = 2 * (x * y - z * w)
    R[:, 0, 2] = 2 * (x * z + y * w)
    R[:, 1, 0] = 2 * (x * y + z * w)
    R[:, 1, 1] = 1 - 2 * (x * x + z * z)
    R[:, 1, 2] = 2 * (y * z - x * w)
    R[:, 2, 0] = 2 * (x * z - y * w)
    R[:, 2, 1] = 2 * (y * z + x * w)
    R[:, 2, 2] = 1 - 2 * (x * x + y * y)
    return R


def _random_walk(rng: np.random.Generator, B: int, N: int, step: float) -> np.ndarray:
    """t_0 = 0, t_{i+1} = t_i + step * u_i with u_i uniform on the unit sphere."""
    u = rng.standard_normal((B, N, 3))
    u /= np.linalg.norm(u, axis=-1, keepdims=True)
    u[:, 0, :] = 0.0
    return step * np.cumsum(u, axis=1)


def _distogram_channels(trans: np.ndarray, R: int, nbins: int = 20, dmax: float = 20.0) -> np.ndarray:
    """One-hot distance bins to the (r+1)-th nearest other residue, computed
    from the full L x L distance matrix (the kNN-distogram preprocessing of the
    FlashIPA rebuttal, paperhub page, answer to Q6).  Returns [B,N,R,nbins]."""
    B, N, _ = trans.shape
    out = np.zeros((B, N, R, nbins))
    width = dmax / nbins
    for b in range(B):
        t = trans[b]
        d2 = np.sum((t[:, None, :] - t[None, :, :]) ** 2, axis=-1)
        np.fill_diagonal(d2, np.inf)
        nn = np.argsort(d2, axis=1)[:, :R]
        for r in range(R):
            d = np.sqrt(d2[np.arange(N), nn[:, r]])
            idx = np.minimum((d / width).astype(np.int64), nbins - 1)
            out[b, np.arange(N), r, idx] = 1.0
    return out


def make_positions(B: int, N: int, seed: int, *, frames: str = "walk", step: float = 3.8,
                   trans_sigma: float = 10.0, box: int = 3, lengths: Optional[tuple] = None,
                   dropout: float = 0.0) -> dict:
    """Seeded residue positions and masks for the kNN distogram.

    frames: "walk" (random walk of `step` angstrom), "gauss" (N(0, trans_sigma^2)),
    "lattice" (integer coordinates uniform in [-box, box]^3: many exact ties and
    duplicates) or "same" (every residue at the origin).
    lengths: (lo, hi) -> per-sample valid prefix L_b ~ U{lo..hi}; dropout: i.i.d.
    probability that a residue inside the prefix is invalid.
    Returns translation [B,N,3] fp32 and mask [B,N] bool."""
    rng = np.random.default_rng(seed)
    if frames == "walk":
        t = _random_walk(rng, B, N, step)
    elif frames == "gauss":
        t = trans_sigma * rng.standard_normal((B, N, 3))
    elif frames == "lattice":
        t = rng.integers(-box, box + 1, size=(B, N, 3)).astype(np.float64)
    elif frames == "same":
        t = np.zeros((B, N, 3))
    else:
        raise ValueError(frames)
    mask = np.ones((B, N), dtype=bool)
    if lengths is not None:
        lo, hi = lengths
        L = rng.integers(lo, hi + 1, size=B)
        for b in range(B):
            mask[b, L[b]:] = False
    if dropout > 0.0:
        mask &= rng.random((B, N)) >= dropout
    return dict(translation=t.astype(np.float32), mask=mask)


def make_inputs(shape: IPAShape, seed: int, *, frames: str = "walk", step: float = 3.8,
                trans_sigma: float = 10.0, lengths: Optional[tuple] = None,
                masked_keys: tuple = (), pair_dropout: float = 0.0,
                empty_row: bool = False, distogram: bool = False,
                eps: float = 1e-8) -> dict:
    """Draw one seeded input set.

    frames: "walk" (random-walk translations of `step` angstrom with random
    rotations) or "gauss" (translations N(0, trans_sigma^2)).
    lengths: (lo, hi) -> per-sample valid length L_b ~ U{lo..hi}, prefix-valid.
    masked_keys: residue indices of sample 0 whose mask is False.
    pair_dropout: i.i.d. probability that pair_mask[b,i,j] is False.
    empty_row: pair_mask[0, L_0 // 2, :] = False (one valid residue with no
    permitted key).
    distogram: the first 20 pair channels of zl and zr are one-hot distance bins.
    Draw order: rot, trans, q, k, v, q_points, k_points, v_points, zl, zr,
    w_pair, point_weight_raw, w_out, masks.
    """
    s = shape
    rng = np.random.default_rng(seed)
    B, N, H = s.B, s.N, s.H
    rot = _quat_rotations(rng, B * N).reshape(B, N, 3, 3)
    if frames == "walk":
        trans = _random_walk(rng, B, N, step)
    elif frames == "gauss":
        trans = trans_sigma * rng.standard_normal((B, N, 3))
    else:
        raise ValueError(frames)
    q = rng.standard_normal((B, N, H, s.D))
    k = rng.standard_normal((B, N, H, s.D))
    v = rng.standard_normal((B, N, H, s.Dv))
    q_points = rng.standard_normal((B, N, H, s.P, 3))
    k_points = rng.standard_normal((B, N, H, s.P, 3))
    v_points = rng.standard_normal((B, N, H, s.Q, 3))
    zl = rng.standard_normal((B, N, s.R, s.Cz))
    zr = rng.standard_normal((B, N, s.R, s.Cz))
    if distogram:
        nb = min(20, s.Cz)
        dg = _distogram_channels(trans, s.R, nbins=20)[..., :nb]
        zl[..., :nb] = dg
        zr[..., :nb] = dg
    w_pair = rng.standard_normal((H, s.Cz)) / math.sqrt(s.R * s.Cz)
    point_weight_raw = rng.standard_normal(H)
    w_out = rng.standard_normal((s.F, s.Cout)) / math.sqrt(s.F)
    b_out = np.zeros(s.Cout)

    mask = np.ones((B, N), dtype=bool)
    if lengths is not None:
        lo, hi = lengths
        L = rng.integers(lo, hi + 1, size=B)
        for b in range(B):
            mask[b, L[b]:] = False
    for j in masked_keys:
        mask[0, j] = False
    pair_mask = None
    if pair_dropout > 0.0 or empty_row:
        pair_mask = rng.random((B, N, N)) >= pair_dropout
        if empty_row:
            L0 = int(mask[0].sum())
            pair_mask[0, L0 // 2, :] = False

    d = s.dtype
    out = dict(q=q, k=k, v=v, q_points=q_points, k_points=k_points, v_points=v_points,
               rotation=rot, translation=trans, point_weight_raw=point_weight_raw,
               w_pair=w_pair, zl=zl, zr=zr, w_out=w_out, b_out=b_out)
    out = {key: round_to(val, d) for key, val in out.items()}
    out["mask"] = mask
    out["pair_mask"] = pair_mask
    out["eps"] = float(eps)
    out["shape"] = s
    return out


# The five workloads: tiny fp32 case, protein-like batch, RNA-like long chain,
# short-chain large batch, long-sequence sweep (one entry per N).
CONFIGS = {
    "tiny": dict(shape=IPAShape(B=1, N=16, H=4, Cz=16, dtype="f32"),
                 kw=dict(frames="gauss", trans_sigma=10.0, masked_keys=(5,))),
    "protein": dict(shape=IPAShape(B=8, N=256, H=8), kw=dict(frames="walk", step=3.8, lengths=(128, 256))),
    "rna": dict(shape=IPAShape(B=1, N=2048, H=8), kw=dict(frames="walk", step=6.0, distogram=True)),
    "short_batch": dict(shape=IPAShape(B=39, N=512, H=12),
                        kw=dict(frames="walk", step=3.8, lengths=(64, 512), pair_dropout=0.05, empty_row=True)),
}
_CONFIG_INDEX = {"tiny": 1, "protein": 2, "rna": 3, "short_batch": 4}

SWEEP_N = (4096, 8192, 16384, 32768)


def sweep_shapes():
    return {f"sweep_{n}": IPAShape(B=1, N=n, H=8) for n in SWEEP_N}


def make_config(name: str, seed: Optional[int] = None) -> dict:
    """Inputs for a named workload; seed defaults to 1000 * config_index + N."""
    if name.startswith("sweep_"):
        n = int(name.split("_")[1])
        shape = IPAShape(B=1, N=n, H=8)
        if seed is None:
            seed = 1000 * 5 + n
        return make_inputs(shape, seed, frames="walk", step=3.8)
    cfg = CONFIGS[name]
    shape = cfg["shape"]
    if seed is None:
        seed = 1000 * _CONFIG_INDEX[name] + shape.N
    return make_inputs(shape, seed, **cfg["kw"])


def make_bias_inputs(B: int, N: int, M: int, H: int, D: int, Dv: int, R: int, seed: int, *,
                     kind: str = "random", dtype: str = "bf16", phi_dtype: str = "f32", masked_keys=(),
                     empty_sample: bool = False,
                     box: float = 1.0, gamma=None) -> dict:
    """Inputs of attention with a low-rank bias: q [B,N,H,D], k [B,M,H,D],
    v [B,M,H,Dv] (standard normal, rounded to `dtype`, "f32" or "bf16"), bias
    factors phi_q [B,N,H,R], phi_k [B,M,H,R] (rounded to `phi_dtype`) and
    key_mask [B,M] (True = permitted).  The factors are inputs here, written out from
    the bias they stand for:

      kind "random": standard normal factors;
      kind "alibi":  R = 2, phi_q(i) = [-m_h i, m_h], phi_k(j) = [1, j] with
                     m_h = 2^(-8 (h+1) / H) (with causal attention this is the
                     ALiBi bias -m_h (i - j));
      kind "sqdist": R = 5, points x_i, y_j uniform in a cube of side `box`,
                     phi_q(i) = [-g_h |x_i|^2, 2 g_h x_i, -g_h],
                     phi_k(j) = [1, y_j, |y_j|^2] (the bias -g_h |x_i - y_j|^2);
                     g_h from `gamma` (default: H values spread over
                     [0.5, 4] / box^2).

    `masked_keys` lists key indices masked in every sample; `empty_sample`
    masks every key of the last sample."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, N, H, D))
    k = rng.standard_normal((B, M, H, D))
    v = rng.standard_normal((B, M, H, Dv))
    if kind == "random":
        pq = rng.standard_normal((B, N, H, R))
        pk = rng.standard_normal((B, M, H, R))
    elif kind == "alibi":
        assert R == 2
        m = 2.0 ** (-8.0 * (np.arange(H) + 1) / H)
        i = np.arange(N, dtype=np.float64)[None, :, None]
        j = np.arange(M, dtype=np.float64)[None, :, None]
        pq = np.stack(np.broadcast_arrays(-m * i, m * np.ones_like(i)), -1)
        pk = np.stack(np.broadcast_arrays(np.ones_like(j) * np.ones(H), j * np.ones(H)), -1)
        pq = np.broadcast_to(pq, (B, N, H, 2))
        pk = np.broadcast_to(pk, (B, M, H, 2))
    elif kind == "sqdist":
        assert R == 5
        x = box * rng.random((B, N, 3))
        y = x[:, :M] if M <= N and N == M else box * rng.random((B, M, 3))
        g = np.asarray(gamma if gamma is not None else np.linspace(0.5, 4.0, H) / box ** 2, np.float64)
        xx = np.sum(x * x, -1)[..., None, None]
        yy = np.sum(y * y, -1)[..., None, None]
        gg = g[None, None, :, None]
        pq = np.concatenate([-gg * xx, 2.0 * gg * x[:, :, None, :], np.broadcast_to(-gg, (B, N, H, 1))], -1)
        pk = np.concatenate([np.ones((B, M, H, 1)), np.broadcast_to(y[:, :, None, :], (B, M, H, 3)),
                             np.broadcast_to(yy, (B, M, H, 1))], -1)
    else:
        raise ValueError(kind)
    km = np.ones((B, M), bool)
    for j0 in masked_keys:
        km[:, j0] = False
    if empty_sample:
        km[-1] = False
    out = {n: round_to(np.ascontiguousarray(a, dtype=np.float32), dtype) for n, a in (("q", q), ("k", k), ("v", v))}
    for n, a in (("phi_q", pq), ("phi_k", pk)):
        out[n] = round_to(np.ascontiguousarray(a, dtype=np.float32), phi_dtype)
    out["key_mask"] = km
    out["dims"] = dict(B=B, N=N, M=M, H=H, D=D, Dv=Dv, R=R, dtype=dtype, phi_dtype=phi_dtype)
    return out
