"""Shared helpers of the GPU tests: run the HIP path, run the oracle on the
same seeded inputs, compare."""
from __future__ import annotations

import sys

import numpy as np

from oracle import ipa_factored

FIELDS = ("update", "local_points", "lse", "empty", "o_scalar", "o_zr", "g")


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


GUARD = 16384        # bytes of sentinel before and after every buffer of a forward
GUARD_BYTE = 0xA5
BUFFERS = ("lifted", "epi_ws", "o", "lse", "update", "local_points")


def add_guards(f, names=BUFFERS):
    """Move the named buffers of `f` into allocations GUARD bytes larger on
    each side, the extra bytes holding GUARD_BYTE; `check_guards` then finds
    any write past either end of a buffer."""
    if not hasattr(f, "_guards"):
        f._guards = []
    for name in names:
        inner, raw, nb = guarded_like(getattr(f, name))
        setattr(f, name, inner)
        f._guards.append((name, raw, nb))
    return f


def guarded_like(buf):
    """A tensor shaped like `buf` inside an allocation with GUARD sentinel
    bytes on each side: (tensor, whole allocation, bytes of the tensor)."""
    import torch
    nb = buf.numel() * buf.element_size()
    raw = torch.full((nb + 2 * GUARD,), GUARD_BYTE, dtype=torch.uint8, device=buf.device)
    return raw[GUARD:GUARD + nb].view(buf.dtype).view(buf.shape), raw, nb


def check_guards(f):
    for name, raw, nb in f._guards:
        before = int((raw[:GUARD] != GUARD_BYTE).sum())
        after = int((raw[GUARD + nb:] != GUARD_BYTE).sum())
        assert before == 0 and after == 0, \
            f"{name}: {before} sentinel bytes before and {after} after the buffer overwritten"


def run_gpu(inp: dict, eps=None):
    """One forward on fresh buffers that are poisoned first (workspace bytes
    0xFF, outputs NaN), so a region the kernels skip, or read unwritten,
    cannot pass on values left behind by an earlier call; every buffer sits
    between two guard bands of sentinel bytes, checked after the forward."""
    import torch
    from rna_structure_amd import _lib
    shape = inp["shape"]
    t = _lib.device_inputs(inp, "cuda")
    f = _lib.FlashIPA(shape, eps=inp["eps"] if eps is None else eps, with_pair_mask=t["pair_mask"] is not None)
    add_guards(f)
    f.poison()
    out = f.forward(t)
    torch.cuda.synchronize()
    check_guards(f)
    return f, t, {k: v.detach().cpu().numpy().astype(np.float64) for k, v in out.items()}


def split_o(o: np.ndarray, shape):
    Dv, RCz, Q = shape.Dv, shape.R * shape.Cz, shape.Q
    B, N, H, _ = o.shape
    return dict(o_scalar=o[..., :Dv], o_zr=o[..., Dv:Dv + RCz].reshape(B, N, H, shape.R, shape.Cz),
                g=o[..., Dv + RCz:].reshape(B, N, H, Q, 3))


def max_abs_rel(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max |ref| (both finite where compared)."""
    denom = np.max(np.abs(ref)) if ref.size else 0.0
    if denom == 0.0:
        return float(np.max(np.abs(got))) if got.size else 0.0
    return float(np.max(np.abs(got - ref)) / denom)


def compare(inp: dict, gpu: dict, rows=None, tol=2e-2, lse_tol=None, verbose=True):
    """Compare the GPU outputs with the oracle on `rows` (all rows if None)."""
    shape = inp["shape"]
    N = shape.N
    rows = np.arange(N) if rows is None else np.asarray(rows)
    ref = ipa_factored(inp, rows=rows, keep=("update", "local_points", "lse", "empty", "o_scalar", "g"))
    got = split_o(gpu["o"], shape)
    errs = {}
    errs["update"] = max_abs_rel(gpu["update"][:, rows], ref["update"])
    errs["local_points"] = max_abs_rel(gpu["local_points"][:, rows], ref["local_points"])
    errs["o_scalar"] = max_abs_rel(got["o_scalar"][:, rows], ref["o_scalar"])
    errs["o_zr"] = max_abs_rel(got["o_zr"][:, rows], ref["o_zr"])
    errs["g"] = max_abs_rel(got["g"][:, rows], ref["g"])
    lse_g = gpu["lse"][:, :, rows]
    lse_r = ref["lse"]
    fin = np.isfinite(lse_r)
    assert np.array_equal(np.isfinite(lse_g), fin), "empty-neighbourhood rows differ"
    errs["lse"] = max_abs_rel(lse_g[fin], lse_r[fin]) if fin.any() else 0.0
    empty = ref["empty"]
    if empty.any():
        bi = np.nonzero(empty)
        assert np.all(gpu["update"][:, rows][bi] == 0.0)
        assert np.all(gpu["local_points"][:, rows][bi] == 0.0)
    for key in ("update", "local_points", "o"):
        assert np.all(np.isfinite(gpu[key])), key
    assert not np.any(np.isnan(gpu["lse"])), "lse"
    if verbose:
        say("  max-abs-rel " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    lt = tol if lse_tol is None else lse_tol
    for k, v in errs.items():
        assert v <= (lt if k == "lse" else tol), f"{k}: {v:.3e} > {tol:.1e}"
    return errs
