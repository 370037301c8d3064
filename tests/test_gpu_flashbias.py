"""GPU parity of attention with a low-rank bias (ipa_bias_attention) against
the float64 oracle (oracle/flashbias_oracle.py) on the same seeded inputs.

Tolerance, from the arithmetic: the query side of every q.k product is
rounded to bf16 (relative 2^-9, a logit error of at most 2^-9 scale sum|q k|,
~1e-2 for D = 64 normal rows), factor products carry ~2^-16 of their
magnitude (bf16 hi/lo pairs), and probabilities are rounded to bf16 against
bf16 values (2^-9).  Bar: max |o - ref| / max |ref| <= 2e-2 per case (the
bf16 bar of the IPA forward), |lse - ref| <= 2e-2 max(1, |ref|), and the same
empty rows (O = 0, lse = -inf).  At the benchmark sizes the oracle computes
sampled rows, tile edges and the last row included.  The workspace is
filled with all-ones bytes (NaN) before every call, so a region the lift
leaves unwritten cannot pass on stale data."""
import numpy as np
import pytest

from oracle import flashbias_attention, flashbias_rows
from rna_structure_amd.synth import make_bias_inputs

from gpu_helpers import add_guards, check_guards, max_abs_rel, say

pytestmark = pytest.mark.gpu


def _run(inp, scale, causal, f=None):
    import torch
    from rna_structure_amd import _lib
    d = inp["dims"]
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}
    dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda").to(dt).contiguous()
    q, k, v = (dev(inp[n], tdt[d["dtype"]]) for n in ("q", "k", "v"))
    pq = dev(inp["phi_q"], tdt[d["phi_dtype"]]) if d["R"] > 0 else None
    pk = dev(inp["phi_k"], tdt[d["phi_dtype"]]) if d["R"] > 0 else None
    km = torch.from_numpy(inp["key_mask"].astype(np.uint8)).cuda()
    if f is None:
        f = _lib.BiasAttention(d["B"], d["N"], d["M"], d["H"], d["D"], d["Dv"], d["R"], scale, causal,
                               d["dtype"], d["phi_dtype"])
        add_guards(f, ("workspace", "o", "lse"))
    # every byte of the workspace that the kernels read must have been written
    # by this call: start from all-ones bytes (NaN as bf16 or fp32)
    f.workspace.fill_(255)
    out = f(q, k, v, pq, pk, km)
    torch.cuda.synchronize()
    check_guards(f)
    return f, {n: t.cpu().numpy().astype(np.float64) for n, t in out.items()}


def _compare(got, ref, rows=None):
    o = got["o"] if rows is None else got["o"][:, rows]
    lse = got["lse"] if rows is None else got["lse"][:, :, rows]
    assert np.array_equal(np.isneginf(lse), np.isneginf(ref["lse"])), "empty rows differ"
    fin = np.isfinite(ref["lse"])
    e_lse = float(np.max(np.abs(lse[fin] - ref["lse"][fin]) / np.maximum(1.0, np.abs(ref["lse"][fin])))) if fin.any() else 0.0
    empty = ~fin.transpose(0, 2, 1)  # [B, N, H]
    assert np.all(o[empty] == 0.0), "empty rows must be zero"
    e_o = max_abs_rel(o, ref["o"])
    say(f"  o max-abs-rel {e_o:.2e}, lse rel {e_lse:.2e}")
    assert e_o <= 2e-2
    assert e_lse <= 2e-2


CASES = [
    # name, dims, seed, kind, causal, generator options
    ("small-random-f32", dict(B=2, N=70, M=70, H=3, D=16, Dv=16, R=2), 1, "random", False,
     dict(dtype="f32", masked_keys=(3, 64), empty_sample=True)),
    ("alibi-causal", dict(B=1, N=300, M=300, H=4, D=64, Dv=64, R=2), 2, "alibi", True, dict()),
    ("sqdist-box10", dict(B=2, N=257, M=257, H=2, D=32, Dv=48, R=5), 3, "sqdist", False, dict(box=10.0)),
    ("cross-ragged", dict(B=2, N=100, M=333, H=2, D=8, Dv=3, R=1), 4, "random", False,
     dict(dtype="f32", masked_keys=(332,))),
    ("widest", dict(B=1, N=130, M=200, H=1, D=128, Dv=256, R=40), 5, "random", False, dict()),
    ("d128", dict(B=1, N=200, M=200, H=2, D=128, Dv=128, R=2), 6, "random", True, dict()),
    ("no-bias", dict(B=1, N=190, M=190, H=2, D=64, Dv=64, R=0), 7, "random", False, dict()),
    ("no-bias-d128", dict(B=1, N=150, M=150, H=1, D=128, Dv=64, R=0), 10, "random", True, dict()),
    ("bf16-factors", dict(B=1, N=129, M=129, H=2, D=32, Dv=32, R=3), 8, "random", False, dict(phi_dtype="bf16")),
    ("one-query", dict(B=1, N=1, M=1, H=1, D=4, Dv=4, R=1), 9, "random", True, dict(dtype="f32")),
    # causal with a batch, masked keys (one of them a query's only causal key) and an empty sample
    ("batch-causal-masks", dict(B=3, N=200, M=200, H=2, D=32, Dv=20, R=3), 12, "random", True,
     dict(dtype="f32", masked_keys=(0, 63, 64, 199), empty_sample=True)),
]


@pytest.mark.parametrize("name,dims,seed,kind,causal,opts", CASES, ids=[c[0] for c in CASES])
def test_bias_attention_matches_oracle(name, dims, seed, kind, causal, opts):
    say(f"case bias attention {name} {dims} causal={causal} {opts}")
    inp = make_bias_inputs(**dims, seed=seed, kind=kind, **opts)
    scale = 1.0 / np.sqrt(dims["D"])
    _, got = _run(inp, scale, causal)
    ref = flashbias_attention(inp["q"], inp["k"], inp["v"], inp["phi_q"], inp["phi_k"], scale,
                              key_mask=inp["key_mask"], causal=causal)
    _compare(got, ref)


@pytest.mark.parametrize("name,dims,kind,causal,opts", [
    ("alibi-gpt2-2048", dict(B=2, N=2048, M=2048, H=25, D=64, Dv=64, R=2), "alibi", True, dict()),
    ("sqdist-pde-32186", dict(B=1, N=32186, M=32186, H=8, D=32, Dv=32, R=5), "sqdist", False, dict()),
], ids=["alibi-gpt2-2048", "sqdist-pde-32186"])
def test_bias_attention_full_size_sampled_rows(name, dims, kind, causal, opts):
    say(f"case bias attention full size {name} {dims}")
    inp = make_bias_inputs(**dims, seed=11, kind=kind, **opts)
    scale = 1.0 / np.sqrt(dims["D"])
    f, got = _run(inp, scale, causal)
    N = dims["N"]
    rows = np.unique(np.array([0, 1, 63, 64, 127, 128, N // 2 + 5, N - 2, N - 1]))
    ref = flashbias_rows(inp["q"], inp["k"], inp["v"], inp["phi_q"], inp["phi_k"], scale, rows,
                         key_mask=inp["key_mask"], causal=causal)
    _compare(got, ref, rows)
    # a second call on the same buffers gives the same bits
    _, again = _run(inp, scale, causal, f)
    assert np.array_equal(again["o"], got["o"]) and np.array_equal(again["lse"], got["lse"])


@pytest.mark.parametrize("causal", [False, True])
def test_weights_applied_to_values_sum_to_one(causal):
    """With every value equal to 1 the output is the sum of the weights the
    value product applies: 1 within fp32 rounding (1e-5) on every non-empty
    row, not just within the bf16 rounding of the weights."""
    dims = dict(B=2, N=300, M=300, H=3, D=32, Dv=16, R=2)
    inp = make_bias_inputs(**dims, seed=13, kind="random", masked_keys=(7, 64, 299), empty_sample=True)
    inp["v"] = np.ones_like(inp["v"])
    say(f"case bias attention unit values causal={causal}")
    _, got = _run(inp, 1.0 / np.sqrt(dims["D"]), causal)
    fin = np.isfinite(got["lse"]).transpose(0, 2, 1)  # [B, N, H]
    assert fin.any() and not fin.all()
    o = got["o"]
    assert np.max(np.abs(o[fin] - 1.0)) <= 1e-5, np.max(np.abs(o[fin] - 1.0))
    assert np.all(o[~fin] == 0.0)
