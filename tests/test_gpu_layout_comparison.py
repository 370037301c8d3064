"""The pages' stacked point layout against this build's, on a long chain.

The FlashIPA rebuttal (paperhub page, Q3) runs FlashAttention-2 on stacked
vectors with five columns per point: the query side holds [T_i q_p,
|T_i q_p|^2, 1] and the key side [2 gamma T_j k_p, -gamma, -gamma |T_j k_p|^2],
so that their inner product is the point term -gamma |T_i q_p - T_j k_p|^2.
With 16-bit operands the squared norms of global coordinates swamp the
result on long chains (bf16), or overflow (fp16, max 65504).  This build
expands about per-tile and per-wavefront centroids with an fp16 hi/lo split
instead; the test measures both against the float64 oracle on the same rows
of an N = 16384 walk and records the errors (the kernel's own logits come
from ipa_logit_rows, the same MFMA sequence as the fused kernel)."""
import math

import numpy as np
import pytest

from oracle import ipa_factored, point_weight, to_global
from rna_structure_amd.synth import IPAShape, make_inputs

from gpu_helpers import run_gpu, say

pytestmark = pytest.mark.gpu


def _round_bf16(x):
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32)


def _round_f16(x):
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)


def test_stacked_point_layout_versus_centred_split():
    s = IPAShape(B=1, N=16384, H=2, dtype="bf16")
    inp = make_inputs(s, 77, frames="walk", step=3.8)
    say(f"case layout comparison {s}")
    f, _, _ = run_gpu(inp)
    rows = np.array([0, 4097, 9000, 16383])
    ref = ipa_factored(inp, rows=rows, keep=("logits",))["logits"]          # [1,H,4,N]
    A = to_global(inp["rotation"], inp["translation"], inp["q_points"])[0, rows]   # [4,H,P,3]
    Bk = to_global(inp["rotation"], inp["translation"], inp["k_points"])[0]        # [N,H,P,3]
    gam = point_weight(inp["point_weight_raw"], s.P)
    errs = {"this build": 0.0, "stacked bf16": 0.0, "stacked fp16": 0.0}
    near = dict(errs)   # over the keys that carry weight: logit within 20 of the row maximum
    scale = 0.0
    for h in range(s.H):
        L = np.stack([f.logit_rows(0, h, int(i), 1).cpu().numpy()[0] for i in rows]).astype(np.float64)
        sel = ref[0, h] > ref[0, h].max(axis=-1, keepdims=True) - 20.0
        errs["this build"] = max(errs["this build"], float(np.max(np.abs(L - ref[0, h]))))
        near["this build"] = max(near["this build"], float(np.max(np.abs(L - ref[0, h])[sel])))
        scale = max(scale, float(np.max(np.abs(ref[0, h]))))
        exact = -gam[h] * np.sum((A[:, None, h] - Bk[None, :, h]) ** 2, axis=(-1, -2))   # [4,N]
        qs = np.concatenate([A[:, h], np.sum(A[:, h] ** 2, -1, keepdims=True), np.ones((4, s.P, 1))], -1)
        ks = np.concatenate([2 * gam[h] * Bk[:, h], -gam[h] * np.ones((s.N, s.P, 1)),
                             -gam[h] * np.sum(Bk[:, h] ** 2, -1, keepdims=True)], -1)
        qs, ks = qs.reshape(4, -1), ks.reshape(s.N, -1)                     # 5P columns
        for name, rnd in (("stacked bf16", _round_bf16), ("stacked fp16", _round_f16)):
            with np.errstate(invalid="ignore", over="ignore"):
                approx = (rnd(qs) @ rnd(ks).T).astype(np.float64)
            e = np.abs(approx - exact)
            e = np.where(np.isfinite(e), e, np.inf)
            errs[name] = max(errs[name], float(np.max(e)))
            near[name] = max(near[name], float(np.max(e[sel])))
    say("  max |logit error| " + ", ".join(f"{k} {v:.3g}" for k, v in errs.items()) + f" (logits up to {scale:.3g})")
    say("  on keys within 20 of the row maximum: " + ", ".join(f"{k} {v:.3g}" for k, v in near.items()))
    assert errs["this build"] <= 5e-2 * max(1.0, scale)
    assert near["this build"] <= 2e-2
    assert near["stacked bf16"] > 100 * near["this build"]
    assert errs["stacked bf16"] > 100 * errs["this build"]
    assert not math.isfinite(errs["stacked fp16"]) or errs["stacked fp16"] > 100 * errs["this build"]
