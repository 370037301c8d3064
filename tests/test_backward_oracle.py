"""Pins of the gradient oracle (oracle/ipa_backward.py) against things other
than itself: the NumPy forward oracle, central finite differences, the
transformation of gradients under a common rigid motion, and torch's own
scaled_dot_product_attention when the point and pair terms are switched off.
"""
import math

import numpy as np
import pytest
import torch

from oracle import ipa_factored
from oracle.ipa_backward import GRAD_KEYS, ipa_forward_torch, ipa_gradients
from rna_structure_amd.synth import IPAShape, make_inputs


def _small(seed=0, B=2, N=7, H=2, **kw):
    s = IPAShape(B=B, N=N, H=H, D=3, Dv=2, P=2, Q=2, Cz=3, R=2, Cout=4, dtype="f32")
    return make_inputs(s, seed, frames="gauss", trans_sigma=2.0, **kw)


def _upstream(inp, seed):
    rng = np.random.default_rng(seed)
    s = inp["shape"]
    return (rng.standard_normal((s.B, s.N, s.Cout)), rng.standard_normal((s.B, s.N, s.H, s.Q, 3)))


def _tensors(inp):
    return {key: torch.tensor(inp[key], dtype=torch.float64) for key in GRAD_KEYS}


def _loss(inp, du, dl):
    t = _tensors(inp)
    pm = inp.get("pair_mask")
    out = ipa_forward_torch(t, torch.tensor(inp["mask"]), None if pm is None else torch.tensor(pm), inp["eps"])
    return float((out["update"].numpy() * du).sum() + (out["local_points"].numpy() * dl).sum())


def test_torch_forward_equals_numpy_oracle():
    inp = _small(1, masked_keys=(3,), pair_dropout=0.2, empty_row=True, lengths=(4, 7))
    t = _tensors(inp)
    out = ipa_forward_torch(t, torch.tensor(inp["mask"]), torch.tensor(inp["pair_mask"]), inp["eps"])
    ref = ipa_factored(inp, keep=("update", "local_points"))
    np.testing.assert_allclose(out["update"].numpy(), ref["update"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(out["local_points"].numpy(), ref["local_points"], rtol=0, atol=1e-12)


@pytest.mark.parametrize("kw", [dict(), dict(masked_keys=(2,), pair_dropout=0.25, empty_row=True, lengths=(5, 7))])
def test_gradients_equal_central_differences(kw):
    """Every input tensor, several random elements each: autograd against
    (f(x+h) - f(x-h)) / 2h in float64."""
    inp = _small(2, **kw)
    du, dl = _upstream(inp, 3)
    grads = ipa_gradients(inp, du, dl)
    rng = np.random.default_rng(4)
    h = 1e-6
    for key in GRAD_KEYS:
        x = inp[key]
        flat = x.reshape(-1)
        for idx in rng.choice(flat.size, size=min(6, flat.size), replace=False):
            old = flat[idx]
            flat[idx] = old + h
            fp = _loss(inp, du, dl)
            flat[idx] = old - h
            fm = _loss(inp, du, dl)
            flat[idx] = old
            fd = (fp - fm) / (2 * h)
            g = grads[key].reshape(-1)[idx]
            assert abs(fd - g) <= 1e-6 * max(1.0, abs(fd)), (key, idx, fd, g)


def _rot(rng):
    qt = rng.standard_normal(4)
    qt /= np.linalg.norm(qt)
    w, x, y, z = qt
    return np.array([[1 - 2 * (y * y + z * z), 2 * (x * y - z * w), 2 * (x * z + y * w)],
                     [2 * (x * y + z * w), 1 - 2 * (x * x + z * z), 2 * (y * z - x * w)],
                     [2 * (x * z - y * w), 2 * (y * z + x * w), 1 - 2 * (x * x + y * y)]])


def test_gradients_under_a_common_rigid_motion():
    """R_i -> G R_i, t_i -> G t_i + u leaves the outputs unchanged, so the
    gradients of every non-frame input are unchanged and the frame gradients
    turn with G: dR' = G dR, dt' = G dt."""
    inp = _small(5, pair_dropout=0.1, empty_row=True)
    du, dl = _upstream(inp, 6)
    g0 = ipa_gradients(inp, du, dl)
    rng = np.random.default_rng(7)
    G, u = _rot(rng), rng.standard_normal(3) * 5
    moved = dict(inp)
    moved["rotation"] = np.einsum("xy,bnyz->bnxz", G, inp["rotation"])
    moved["translation"] = np.einsum("xy,bny->bnx", G, inp["translation"]) + u
    g1 = ipa_gradients(moved, du, dl)
    for key in GRAD_KEYS:
        if key in ("rotation", "translation"):
            continue
        np.testing.assert_allclose(g1[key], g0[key], rtol=1e-9, atol=1e-10, err_msg=key)
    np.testing.assert_allclose(g1["rotation"], np.einsum("xy,bnyz->bnxz", G, g0["rotation"]), rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(g1["translation"], np.einsum("xy,bny->bnx", G, g0["translation"]), rtol=1e-9,
                               atol=1e-10)
    # a common translation changes nothing: the translation gradients sum to zero
    np.testing.assert_allclose(g0["translation"].sum(axis=1), 0.0, atol=1e-10)


def test_reduces_to_scaled_dot_product_attention():
    """Point weight ~ 0 (softplus(-60)), no pair bias, w_out reading only the
    scalar features: the q, k, v gradients are those of plain attention with
    scale 1/sqrt(3D), from torch's own implementation."""
    inp = _small(8, B=1, N=6, H=1)
    s = inp["shape"]
    inp["point_weight_raw"] = np.full(s.H, -60.0)
    inp["w_pair"] = np.zeros_like(inp["w_pair"])
    w = np.zeros_like(inp["w_out"])
    rng = np.random.default_rng(9)
    w[: s.H * s.Dv] = rng.standard_normal((s.H * s.Dv, s.Cout))
    inp["w_out"] = w
    du, dl = _upstream(inp, 10)
    dl[:] = 0.0
    grads = ipa_gradients(inp, du, dl, keys=("q", "k", "v"))
    q = torch.tensor(inp["q"], dtype=torch.float64, requires_grad=True)
    k = torch.tensor(inp["k"], dtype=torch.float64, requires_grad=True)
    v = torch.tensor(inp["v"], dtype=torch.float64, requires_grad=True)
    o = torch.nn.functional.scaled_dot_product_attention(
        q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2), scale=1.0 / math.sqrt(3.0 * s.D))
    upd = o.transpose(1, 2).reshape(1, s.N, -1) @ torch.tensor(w[: s.H * s.Dv]) + torch.tensor(inp["b_out"])
    (upd * torch.tensor(du)).sum().backward()
    for key, ref in (("q", q.grad), ("k", k.grad), ("v", v.grad)):
        np.testing.assert_allclose(grads[key], ref.numpy(), rtol=1e-10, atol=1e-12, err_msg=key)


def test_empty_rows_pass_no_gradient():
    """Upstream gradients on an empty row change no input gradient."""
    inp = _small(11, empty_row=True)
    du, dl = _upstream(inp, 12)
    g0 = ipa_gradients(inp, du, dl)
    b, i = 0, int(inp["mask"][0].sum()) // 2        # the empty row of synth's recipe
    assert not inp["pair_mask"][b, i].any()
    du2, dl2 = du.copy(), dl.copy()
    du2[b, i] += 3.0
    dl2[b, i] -= 2.0
    g1 = ipa_gradients(inp, du2, dl2)
    for key in GRAD_KEYS:
        np.testing.assert_allclose(g1[key], g0[key], rtol=0, atol=1e-12, err_msg=key)


def test_row_restricted_gradients_equal_full_with_zero_upstream_elsewhere():
    """The row-restricted forward (only the selected query rows, against all
    keys) gives the full oracle's gradients when the upstream gradients of
    every other row are zero: masks, a pair mask and the empty row included,
    rows in any order, a repeated row counted twice."""
    inp = _small(13, B=2, N=9, H=3, masked_keys=(2,), pair_dropout=0.2, empty_row=True)
    du, dl = _upstream(inp, 14)
    for rows in ([0, 4, 8], [7, 1], [3, 3, 5]):
        du_full, dl_full = np.zeros_like(du), np.zeros_like(dl)
        for k, i in enumerate(rows):
            du_full[:, i] += du[:, k]
            dl_full[:, i] += dl[:, k]
        g_full = ipa_gradients(inp, du_full, dl_full)
        g_rows = ipa_gradients(inp, du[:, :len(rows)], dl[:, :len(rows)], rows=rows)
        for key in GRAD_KEYS:
            np.testing.assert_allclose(g_rows[key], g_full[key], rtol=1e-12, atol=1e-13, err_msg=f"{rows} {key}")
    # the restricted forward's outputs are the full forward's rows
    t = _tensors(inp)
    mask = torch.tensor(inp["mask"], dtype=torch.bool)
    pm = torch.tensor(inp["pair_mask"], dtype=torch.bool)
    full = ipa_forward_torch(t, mask, pm, inp["eps"])
    part = ipa_forward_torch(t, mask, pm, inp["eps"], rows=[8, 2, 5])
    for key in ("update", "local_points"):
        np.testing.assert_allclose(part[key].detach().numpy(), full[key].detach().numpy()[:, [8, 2, 5]],
                                   rtol=1e-13, atol=1e-14)
