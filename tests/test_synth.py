"""Seeded input generator: shapes, determinism, rounding, mask recipes."""
import numpy as np
import torch

from rna_structure_amd.synth import CONFIGS, IPAShape, make_config, make_inputs, round_to


def test_deterministic():
    a = make_config("protein")
    b = make_config("protein")
    for key in ("q", "rotation", "translation", "zl", "mask"):
        np.testing.assert_array_equal(a[key], b[key])


def test_bf16_rounding_is_exact_and_rne():
    x = np.random.default_rng(0).standard_normal(10000) * 100
    r = round_to(x, "bf16")
    t = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(r, t)


def test_config_recipes():
    p = make_config("protein")
    L = p["mask"].sum(1)
    assert p["q"].shape == (8, 256, 8, 16) and np.all((L >= 128) & (L <= 256))
    for b in range(8):
        assert p["mask"][b, :L[b]].all() and not p["mask"][b, L[b]:].any()
    steps = np.linalg.norm(np.diff(p["translation"][0], axis=0), axis=-1)
    assert np.all(np.abs(steps - 3.8) < 0.6) and abs(steps.mean() - 3.8) < 0.05   # bf16-rounded 3.8 A steps
    rot = p["rotation"][0, 0]
    assert abs(np.linalg.det(rot) - 1) < 2e-2
    s = make_config("short_batch")
    L0 = int(s["mask"][0].sum())
    assert not s["pair_mask"][0, L0 // 2].any()
    assert 0.93 < s["pair_mask"].mean() < 0.97
    t = make_config("tiny")
    assert t["shape"].dtype == "f32" and not t["mask"][0, 5] and t["mask"].sum() == 15


def test_distogram_channels_one_hot():
    s = IPAShape(B=1, N=64, H=2)
    x = make_inputs(s, 3, frames="walk", step=6.0, distogram=True)
    dg = x["zl"][0, :, :, :20]
    assert np.all(dg.sum(-1) == 1.0)
    np.testing.assert_array_equal(x["zl"][..., :20], x["zr"][..., :20])
