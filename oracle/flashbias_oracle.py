"""Plain CPU oracle of attention with a low-rank bias (FlashBias).

TEST INFRASTRUCTURE ONLY.  This file is imported by tests/, by
__graft_entry__.smoke() and by the cpu_baseline leg of bench.py, and by
nothing else.  It shares no code with the HIP library and does not import it.

What it computes (FlashBias: Fast Computation of Attention with Bias,
atlas.scime.ai summary, Problem and Approach): attention whose logits carry an
additive bias b_ij, where the dense [N, M] bias is replaced by two factor
tensors with b_ij = phi_q(i) . phi_k(j); the factors are concatenated onto
the queries and keys, so that the biased attention is plain attention over
the widened rows:

    L_ij = scale q_i . k_j + phi_q(i) . phi_k(j)
         = [scale q_i | phi_q(i)] . [k_j | phi_k(j)]
    O_i  = sum_j softmax_j(L_ij) v_j,   lse_i = log sum_j exp(L_ij)

over the permitted keys j (key mask, and j <= i when causal).  The page names
exact factors for ALiBi and for a squared-distance bias; their formulas are
not printed, so the readings taken here are the standard definitions:

  * ALiBi (causal): b_ij = -m_h (i - j) for j <= i, head slopes
    m_h = 2^(-8 (h + 1) / H); exact rank-2 factors
    phi_q(i) = [-m_h i, m_h], phi_k(j) = [1, j];
  * squared distance: b_ij = -gamma |x_i - y_j|^2; exact rank-5 factors
    phi_q(i) = [-gamma |x_i|^2, 2 gamma x_i, -gamma], phi_k(j) = [1, y_j, |y_j|^2].

A row with no permitted key gets O_i = 0 and lse_i = -inf (the convention of
the IPA kernels of this library).  Float64 throughout.

Pins (tests/test_flashbias_oracle.py): the dense form against torch's
scaled_dot_product_attention with an additive mask (library routine), the
factor products against the biases written from their definitions
(scipy's cdist for the distances), pure-Python loops on a tiny case, the
causal first row (it sees key 0 only), and the invariance of O under a
bias that is constant along a row.
"""
from __future__ import annotations

import numpy as np


def alibi_slopes(H: int) -> np.ndarray:
    """Head slopes m_h = 2^(-8 (h + 1) / H)."""
    return 2.0 ** (-8.0 * (np.arange(H) + 1) / H)


def alibi_bias(N: int, H: int) -> np.ndarray:
    """Dense ALiBi bias [H, N, N]: -m_h (i - j) (the causal mask is separate)."""
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    return -alibi_slopes(H)[:, None, None] * (i - j)[None].astype(np.float64)


def alibi_factors(B: int, N: int, H: int):
    """Exact rank-2 factors of the ALiBi bias, shaped [B, N, H, 2] each."""
    m = alibi_slopes(H)
    i = np.arange(N, dtype=np.float64)
    pq = np.stack([-m[None, :] * i[:, None], np.broadcast_to(m[None, :], (N, H))], -1)     # [N,H,2]
    pk = np.stack([np.ones((N, H)), np.broadcast_to(i[:, None], (N, H))], -1)
    return (np.broadcast_to(pq, (B, N, H, 2)).copy(), np.broadcast_to(pk, (B, N, H, 2)).copy())


def sqdist_factors(x: np.ndarray, y: np.ndarray, gamma: np.ndarray):
    """Exact rank-5 factors of b_ij = -gamma_h |x_i - y_j|^2.

    x [B, N, 3] query positions, y [B, M, 3] key positions, gamma [H];
    returns phi_q [B, N, H, 5], phi_k [B, M, H, 5]."""
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    g = np.asarray(gamma, np.float64)
    B, N, _ = x.shape
    M = y.shape[1]
    H = g.shape[0]
    xx = np.sum(x * x, -1)
    yy = np.sum(y * y, -1)
    pq = np.concatenate([(-g[None, None, :] * xx[:, :, None])[..., None],
                         2.0 * g[None, None, :, None] * x[:, :, None, :],
                         np.broadcast_to(-g[None, None, :, None], (B, N, H, 1))], -1)
    pk = np.concatenate([np.ones((B, M, H, 1)),
                         np.broadcast_to(y[:, :, None, :], (B, M, H, 3)),
                         np.broadcast_to(yy[:, :, None, None], (B, M, H, 1))], -1)
    return pq, pk


def permitted(B: int, N: int, M: int, key_mask=None, causal: bool = False) -> np.ndarray:
    """Boolean [B, N, M]: key j may be attended by query i."""
    ok = np.ones((B, N, M), bool)
    if key_mask is not None:
        ok &= np.asarray(key_mask, bool)[:, None, :]
    if causal:
        ok &= (np.arange(M)[None, :] <= np.arange(N)[:, None])[None]
    return ok


def softmax_rows(logits: np.ndarray, ok: np.ndarray, v: np.ndarray):
    """O and lse of masked softmax attention.

    logits [B, H, N, M], ok [B, N, M] (broadcast over heads), v [B, M, H, Dv];
    returns o [B, N, H, Dv] and lse [B, H, N]."""
    okh = ok[:, None]
    L = np.where(okh, logits, -np.inf)
    mx = np.max(L, axis=-1, keepdims=True)
    empty = ~np.isfinite(mx)
    e = np.where(okh, np.exp(L - np.where(empty, 0.0, mx)), 0.0)
    s = np.sum(e, axis=-1, keepdims=True)
    p = np.where(empty, 0.0, e / np.where(empty, 1.0, s))
    o = np.einsum("bhij,bjhc->bihc", p, np.asarray(v, np.float64))
    lse = np.where(empty[..., 0], -np.inf, mx[..., 0] + np.log(np.where(empty[..., 0], 1.0, s[..., 0])))
    return o, lse


def attention_with_bias(q, k, v, bias, scale, key_mask=None, causal=False):
    """Dense definition: L = scale q k^T + bias, bias broadcastable to [B, H, N, M]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    B, N, H, _ = q.shape
    M = k.shape[1]
    logits = scale * np.einsum("bihd,bjhd->bhij", q, k) + np.broadcast_to(np.asarray(bias, np.float64), (B, H, N, M))
    return softmax_rows(logits, permitted(B, N, M, key_mask, causal), v)


def flashbias_attention(q, k, v, phi_q, phi_k, scale, key_mask=None, causal=False):
    """Concatenated form: plain attention over [scale q | phi_q] and [k | phi_k].

    q [B, N, H, D], k [B, M, H, D], v [B, M, H, Dv], phi_q [B, N, H, R],
    phi_k [B, M, H, R], key_mask [B, M] or None; returns dict(o, lse)."""
    qq = np.concatenate([scale * np.asarray(q, np.float64), np.asarray(phi_q, np.float64)], -1)
    kk = np.concatenate([np.asarray(k, np.float64), np.asarray(phi_k, np.float64)], -1)
    B, N, H, _ = qq.shape
    M = kk.shape[1]
    logits = np.einsum("bihd,bjhd->bhij", qq, kk)
    o, lse = softmax_rows(logits, permitted(B, N, M, key_mask, causal), v)
    return {"o": o, "lse": lse}


def flashbias_rows(q, k, v, phi_q, phi_k, scale, rows, key_mask=None, causal=False):
    """flashbias_attention restricted to query rows `rows` (for long inputs)."""
    rows = np.asarray(rows)
    q = np.asarray(q)[:, rows]
    pq = np.asarray(phi_q)[:, rows]
    qq = np.concatenate([scale * q.astype(np.float64), pq.astype(np.float64)], -1)
    kk = np.concatenate([np.asarray(k, np.float64), np.asarray(phi_k, np.float64)], -1)
    B, M = kk.shape[0], kk.shape[1]
    ok = np.ones((B, len(rows), M), bool)
    if key_mask is not None:
        ok &= np.asarray(key_mask, bool)[:, None, :]
    if causal:
        ok &= (np.arange(M)[None, :] <= rows[:, None])[None]
    logits = np.einsum("bihd,bjhd->bhij", qq, kk)
    o, lse = softmax_rows(logits, ok, v)
    return {"o": o, "lse": lse}


def attention_loops(q, k, v, bias, scale, key_mask=None, causal=False):
    """The dense definition as pure-Python loops (tiny inputs only)."""
    import math
    B, N, H, D = np.shape(q)
    M, Dv = np.shape(k)[1], np.shape(v)[3]
    o = np.zeros((B, N, H, Dv))
    lse = np.full((B, H, N), -np.inf)
    for b in range(B):
        for h in range(H):
            for i in range(N):
                logit = {}
                for j in range(M):
                    if key_mask is not None and not key_mask[b][j]:
                        continue
                    if causal and j > i:
                        continue
                    logit[j] = scale * sum(float(q[b][i][h][d]) * float(k[b][j][h][d]) for d in range(D)) + float(bias[b][h][i][j])
                if not logit:
                    continue
                mx = max(logit.values())
                tot = sum(math.exp(x - mx) for x in logit.values())
                lse[b, h, i] = mx + math.log(tot)
                for j, x in logit.items():
                    w = math.exp(x - mx) / tot
                    for c in range(Dv):
                        o[b, i, h, c] += w * float(v[b][j][h][c])
    return o, lse
