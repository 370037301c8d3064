"""bf16 against fp16 matrix operands for the scalar and pair columns.

The fused kernel feeds the scalar and pair columns to bf16 MFMAs: the key
side (k, zr) is then exact (the inputs are bf16) and only the query side,
q log2(e)/sqrt(3D) and w_pair zl log2(e)/sqrt(3), is rounded (8 significant
bits).  fp16 operands (11 bits, same MFMA rate on these matrix cores) would
round the query side 4x more finely but re-round the key side, and fail
outright for inputs beyond the fp16 range.  This CPU study measures the
logit error of both schemes against float64 on the standard shape's inputs
(the point term is not involved: it uses its own fp16 hi/lo columns).
"""
import math

import numpy as np

from rna_structure_amd.synth import IPAShape, make_inputs


def _round_bf16(x):
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _round_f16(x):
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def _scalar_pair_logits(q, k, zl, zr, w, D, rq, rk):
    """Scalar + pair logit in log2 units with the query side rounded by rq and
    the key side by rk, products summed in float64 (the MFMA accumulates in
    fp32; its rounding is far below either operand rounding)."""
    l2e = 1.0 / math.log(2.0)
    qs = rq(q * l2e / math.sqrt(3.0 * D))
    ps = rq(w[None, None, :] * zl * l2e / math.sqrt(3.0))         # [N,R,Cz]
    return qs @ rk(k).T + np.einsum("irc,jrc->ij", ps, rk(zr))


def test_bf16_and_fp16_operand_schemes():
    s = IPAShape(B=1, N=512, H=1, dtype="bf16")
    inp = make_inputs(s, 21, frames="walk")
    q, k = inp["q"][0, :, 0], inp["k"][0, :, 0]
    zl, zr, w = inp["zl"][0], inp["zr"][0], inp["w_pair"][0]
    exact = _scalar_pair_logits(q, k, zl, zr, w, s.D, lambda x: x, lambda x: x)
    err = {}
    for name, rq, rk in (("bf16", _round_bf16, lambda x: x), ("fp16", _round_f16, _round_f16)):
        err[name] = float(np.max(np.abs(_scalar_pair_logits(q, k, zl, zr, w, s.D, rq, rk) - exact)))
    print(f"max |logit error| (log2 units) of the scalar + pair part: bf16 {err['bf16']:.2e}, fp16 {err['fp16']:.2e}")
    # bf16 rounds the query side to 2^-9 relative, fp16 to 2^-11
    assert err["fp16"] < err["bf16"] / 2
    assert err["bf16"] < 2e-2
    # fp16 cannot hold a bf16 input of magnitude 1e5 (bf16 can, exactly)
    assert not np.isfinite(_round_f16(np.array([1e5]))[0]) and _round_bf16(np.array([1e5]))[0] == 99840.0
