"""Pins of the low-rank-bias attention oracle (oracle/flashbias_oracle.py).

Each check ties the oracle to something other than itself: torch's
scaled_dot_product_attention with an additive mask (the dense definition),
the ALiBi and squared-distance biases written from their definitions (scipy's
cdist for the distances), pure-Python loops, the causal first row, and the
invariance of the output under a bias that is constant along a row."""
import numpy as np
import pytest
from scipy.spatial.distance import cdist

from oracle import (alibi_bias, alibi_factors, alibi_slopes, attention_loops, attention_with_bias,
                    flashbias_attention, flashbias_rows, sqdist_factors)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_dense_form_matches_torch_sdpa():
    import torch
    rng = np.random.default_rng(1)
    B, N, M, H, D, Dv = 2, 7, 9, 3, 5, 4
    q, k, v = _rand(rng, B, N, H, D), _rand(rng, B, M, H, D), _rand(rng, B, M, H, Dv)
    bias = 2.0 * _rand(rng, B, H, N, M)
    km = rng.random((B, M)) > 0.3
    km[:, 0] = True
    scale = 0.37
    o, lse = attention_with_bias(q, k, v, bias, scale, key_mask=km)
    add = np.where(km[:, None, None, :], bias, -np.inf)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x.transpose(0, 2, 1, 3)))
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=torch.from_numpy(add),
                                                           scale=scale).numpy().transpose(0, 2, 1, 3)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
    L = scale * np.einsum("bihd,bjhd->bhij", q, k) + add
    np.testing.assert_allclose(lse, np.log(np.sum(np.exp(L), -1)), rtol=1e-12, atol=1e-12)


def test_dense_form_matches_loops_with_causal_and_mask():
    rng = np.random.default_rng(2)
    B, N, H, D, Dv = 2, 4, 2, 3, 2
    q, k, v = _rand(rng, B, N, H, D), _rand(rng, B, N, H, D), _rand(rng, B, N, H, Dv)
    bias = _rand(rng, B, H, N, N)
    km = np.array([[True, False, True, True], [False, True, True, True]])
    o, lse = attention_with_bias(q, k, v, bias, 0.5, key_mask=km, causal=True)
    ol, ll = attention_loops(q, k, v, bias, 0.5, key_mask=km, causal=True)
    np.testing.assert_allclose(o, ol, rtol=1e-12, atol=1e-12)
    assert np.array_equal(np.isneginf(lse), np.isneginf(ll))
    fin = np.isfinite(ll)
    np.testing.assert_allclose(lse[fin], ll[fin], rtol=1e-12)
    # sample 1, query 0: its only causal key (0) is masked out -> empty row
    assert np.isneginf(lse[1, :, 0]).all() and np.all(o[1, 0] == 0.0)


def test_alibi_factors_are_exact():
    B, N, H = 1, 300, 6
    pq, pk = alibi_factors(B, N, H)
    prod = np.einsum("bihr,bjhr->bhij", pq, pk)
    i, j = np.meshgrid(np.arange(N), np.arange(N), indexing="ij")
    for h, m in enumerate(alibi_slopes(H)):
        np.testing.assert_allclose(prod[0, h], -m * (i - j), rtol=1e-14, atol=1e-12)
    np.testing.assert_allclose(prod[0], alibi_bias(N, H), rtol=1e-14, atol=1e-12)
    assert alibi_slopes(8)[0] == 0.5 and alibi_slopes(8)[-1] == 2.0 ** -8


def test_sqdist_factors_are_exact():
    rng = np.random.default_rng(3)
    x, y = 3.0 * _rand(rng, 2, 11, 3), 3.0 * _rand(rng, 2, 13, 3)
    g = np.array([0.1, 0.7, 2.0])
    pq, pk = sqdist_factors(x, y, g)
    prod = np.einsum("bihr,bjhr->bhij", pq, pk)
    for b in range(2):
        d2 = cdist(x[b], y[b], "sqeuclidean")
        for h in range(3):
            np.testing.assert_allclose(prod[b, h], -g[h] * d2, rtol=1e-12, atol=1e-10)


@pytest.mark.parametrize("kind", ["alibi", "sqdist"])
def test_concatenated_form_equals_dense_bias(kind):
    rng = np.random.default_rng(4)
    B, N, H, D, Dv = 2, 40, 4, 8, 6
    q, k, v = _rand(rng, B, N, H, D), _rand(rng, B, N, H, D), _rand(rng, B, N, H, Dv)
    if kind == "alibi":
        pq, pk = alibi_factors(B, N, H)
        bias, causal = alibi_bias(N, H)[None], True
    else:
        x = 2.0 * _rand(rng, B, N, 3)
        g = np.array([0.05, 0.2, 0.5, 1.0])
        pq, pk = sqdist_factors(x, x, g)
        bias = -g[None, :, None, None] * np.stack([cdist(x[b], x[b], "sqeuclidean") for b in range(B)])[:, None]
        causal = False
    km = np.ones((B, N), bool)
    km[1, 30:] = False
    f = flashbias_attention(q, k, v, pq, pk, 1 / np.sqrt(D), key_mask=km, causal=causal)
    o, lse = attention_with_bias(q, k, v, bias, 1 / np.sqrt(D), key_mask=km, causal=causal)
    np.testing.assert_allclose(f["o"], o, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(f["lse"], lse, rtol=1e-10, atol=1e-10)
    rows = np.array([0, 17, 39])
    r = flashbias_rows(q, k, v, pq, pk, 1 / np.sqrt(D), rows, key_mask=km, causal=causal)
    np.testing.assert_allclose(r["o"], o[:, rows], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["lse"], lse[:, :, rows], rtol=1e-12)


def test_causal_first_row_sees_key_zero_only():
    rng = np.random.default_rng(5)
    B, N, H, D, Dv = 1, 6, 2, 4, 3
    q, k, v = _rand(rng, B, N, H, D), _rand(rng, B, N, H, D), _rand(rng, B, N, H, Dv)
    pq, pk = _rand(rng, B, N, H, 2), _rand(rng, B, N, H, 2)
    f = flashbias_attention(q, k, v, pq, pk, 0.3, causal=True)
    np.testing.assert_allclose(f["o"][:, 0], v[:, 0], rtol=1e-14)
    expect = 0.3 * np.sum(q[0, 0] * k[0, 0], -1) + np.sum(pq[0, 0] * pk[0, 0], -1)
    np.testing.assert_allclose(f["lse"][0, :, 0], expect, rtol=1e-14)


def test_row_constant_bias_only_shifts_lse():
    rng = np.random.default_rng(6)
    B, N, H, D, Dv = 1, 12, 2, 4, 3
    q, k, v = _rand(rng, B, N, H, D), _rand(rng, B, N, H, D), _rand(rng, B, N, H, Dv)
    c = 5.0 * _rand(rng, B, N, H, 1)
    f0 = flashbias_attention(q, k, v, np.zeros((B, N, H, 1)), np.zeros((B, N, H, 1)), 0.5)
    f1 = flashbias_attention(q, k, v, c, np.ones((B, N, H, 1)), 0.5)
    np.testing.assert_allclose(f1["o"], f0["o"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(f1["lse"], f0["lse"] + c[..., 0].transpose(0, 2, 1), rtol=1e-12)


def test_synthetic_factors_are_the_oracle_biases():
    """The input generator's ALiBi and squared-distance factors are the biases
    the oracle's factor functions define (so GPU cases test those biases)."""
    from rna_structure_amd.synth import make_bias_inputs
    inp = make_bias_inputs(1, 50, 50, 3, 4, 4, 2, seed=1, kind="alibi")
    pq, pk = alibi_factors(1, 50, 3)
    np.testing.assert_allclose(np.einsum("bihr,bjhr->bhij", inp["phi_q"], inp["phi_k"]),
                               np.einsum("bihr,bjhr->bhij", pq, pk), rtol=1e-6, atol=1e-5)
    inp = make_bias_inputs(2, 30, 30, 2, 4, 4, 5, seed=2, kind="sqdist", box=5.0, phi_dtype="f32")
    prod = np.einsum("bihr,bjhr->bhij", inp["phi_q"], inp["phi_k"])
    # recover the points from the key factors and compare with the definition
    y = inp["phi_k"][:, :, 0, 1:4]
    g = -inp["phi_q"][0, 0, :, 4]
    for b in range(2):
        d2 = cdist(y[b], y[b], "sqeuclidean")
        for h in range(2):
            np.testing.assert_allclose(prod[b, h], -g[h] * d2, rtol=1e-4, atol=1e-3 * g[h] * 75)
