"""C-ABI library: loads, exports what include/flashipa.h declares, and the
host-side argument validation (runs without a GPU: invalid arguments are
rejected before any HIP call)."""
import ctypes
import os
import re

import pytest

from rna_structure_amd import _lib
from rna_structure_amd.synth import IPAShape

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flashipa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from rna_structure_amd import build
        build.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ipa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("ipa_lift", "ipa_flash_fwd", "ipa_epilogue"):
        assert n in names


def test_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(_lib.EXPORTS)


def test_version_and_status_strings(lib):
    assert lib.ipa_version().startswith(b"flashipa")
    for code in range(8):
        assert lib.ipa_status_string(code) != b"unknown status"
    assert lib.ipa_status_string(99) == b"unknown status"


def test_struct_sizes_match_c():
    assert ctypes.sizeof(_lib.IpaShape) == 88
    assert ctypes.sizeof(_lib.IpaLiftIn) == 14 * 8
    assert ctypes.sizeof(_lib.IpaEpiIn) == 5 * 8


def _shape(**kw):
    base = dict(B=2, N=300, H=8, D=16, Dv=16, P=4, Q=8, Cz=64, R=2, Cout=128, dtype="bf16")
    base.update(kw)
    return _lib.make_shape(IPAShape(**base))


def test_lifted_bytes_linear_in_n_without_pair_mask(lib):
    # linear where the grid fills the GPU without splitting the keys
    b1 = _lib.lifted_bytes(_shape(N=8192, B=1), False)
    b2 = _lib.lifted_bytes(_shape(N=16384, B=1), False)
    assert b1 > 0 and 1.9 < b2 / b1 < 2.1
    # O(N) everywhere: smaller N add the key-range partial results (at most
    # 4 records of the attention output per query and head, 4 (DO + 4) 4 H
    # bytes per residue), never anything quadratic
    per_res = [_lib.lifted_bytes(_shape(N=n, B=1), False) / n for n in (1024, 2048, 4096, 8192, 16384, 32768)]
    assert max(per_res) - min(per_res) <= 4 * (16 + 128 + 24 + 4) * 4 * 8 + 64, per_res
    with_pm = _lib.lifted_bytes(_shape(N=4096, B=1), True)
    assert with_pm - _lib.lifted_bytes(_shape(N=4096, B=1), False) >= 4096 * 64 * 8


def test_lifted_bytes_rejects(lib):
    assert _lib.lifted_bytes(_shape(N=0), False) == 0
    assert _lib.lifted_bytes(_shape(H=-1), False) == 0
    assert _lib.lifted_bytes(_shape(P=6), False) == 0          # beyond compiled point columns
    assert _lib.lifted_bytes(_shape(Cz=200), False) == 0       # beyond the widest mfma instance
    s = _shape()
    s.dtype = 7
    assert _lib.lifted_bytes(s, False) == 0
    assert _lib.lifted_bytes(_shape(dtype="f32"), False) > 0


def test_o_width(lib):
    assert _lib.o_width(_shape()) == 16 + 2 * 64 + 3 * 8


def test_validation_before_launch(lib):
    s = _shape()
    li = _lib.IpaLiftIn()
    # NULL arguments
    assert lib.ipa_lift(None, ctypes.byref(li), 256, 1 << 30, None) == 1
    assert lib.ipa_lift(ctypes.byref(s), ctypes.byref(li), 256, 1 << 30, None) == 1
    # misaligned pointers (never dereferenced: validation fails first)
    fields = [n for n, _ in _lib.IpaLiftIn._fields_ if n != "pair_mask"]
    li2 = _lib.IpaLiftIn(**{n: 4096 for n in fields})
    li2.q = 4100
    assert lib.ipa_lift(ctypes.byref(s), ctypes.byref(li2), 4096, 1 << 40, None) == 4
    # workspace too small
    li3 = _lib.IpaLiftIn(**{n: 4096 for n in fields})
    assert lib.ipa_lift(ctypes.byref(s), ctypes.byref(li3), 4096, 16, None) == 2
    # shape errors
    bad = _shape(N=0)
    assert lib.ipa_lift(ctypes.byref(bad), ctypes.byref(li3), 4096, 1 << 40, None) == 2
    eps0 = _shape()
    eps0.eps = 0.0
    assert lib.ipa_flash_fwd(ctypes.byref(eps0), 4096, 4096, 4096, None) == 2
    assert lib.ipa_flash_fwd(ctypes.byref(_shape(P=9)), 4096, 4096, 4096, None) == 3
    assert lib.ipa_flash_fwd(ctypes.byref(s), None, 4096, 4096, None) == 1
    assert lib.ipa_flash_fwd(ctypes.byref(s), 4096, 4100, 4096, None) == 4
    ei = _lib.IpaEpiIn(4096, 4096, 4096, 4096, None)
    assert lib.ipa_epilogue(ctypes.byref(s), 4096, 1 << 30, 4096, 4096, ctypes.byref(ei), 4096, 4096, None) == 1
    ei2 = _lib.IpaEpiIn(4096, 4096, 4096, 4096, 4096)
    # the bf16 path needs the epilogue workspace (packed w_out)
    assert lib.ipa_epilogue(ctypes.byref(s), None, 1 << 30, 4096, 4096, ctypes.byref(ei2), 4096, 4096, None) == 1
    assert lib.ipa_epilogue(ctypes.byref(s), 4096, 1 << 30, None, 4096, ctypes.byref(ei2), 4096, 4096, None) == 1
    assert lib.ipa_epilogue(ctypes.byref(s), 4096, 1 << 30, 4100, 4096, ctypes.byref(ei2), 4096, 4096, None) == 4
    assert lib.ipa_epilogue(ctypes.byref(s), 4104, 1 << 30, 4096, 4096, ctypes.byref(ei2), 4096, 4096, None) == 4
    need = lib.ipa_epilogue_workspace_bytes(ctypes.byref(s))
    assert need >= 8 * 128 * 120 * 2        # per-head packed w_out at H=8, Cout=128
    assert lib.ipa_epilogue(ctypes.byref(s), 4096, need - 1, 4096, 4096, ctypes.byref(ei2), 4096, 4096, None) == 2
    # F = 40*(16+32+56) = 4160 with non-standard dimensions: beyond the LDS
    # staging of the general epilogue (the per-head path takes any H, but only
    # Dv=16, Q=8, Cz=64, R=2)
    big = _shape(H=40, Cz=56)
    assert lib.ipa_epilogue_workspace_bytes(ctypes.byref(big)) == 0
    assert lib.ipa_epilogue(ctypes.byref(big), 4096, 1 << 30, 4096, 4096, ctypes.byref(ei2), 4096, 4096, None) == 3
    # the fp32 path packs nothing: no workspace needed
    f32 = _shape(dtype="f32", N=100, H=4)
    assert lib.ipa_epilogue_workspace_bytes(ctypes.byref(f32)) == 16
    assert lib.ipa_logit_rows(ctypes.byref(s), 4096, 5, 0, 0, 1, 4096, None) == 2   # b out of range
    assert lib.ipa_logit_rows(ctypes.byref(s), 4096, 0, 0, 299, 2, 4096, None) == 2  # rows past N


def test_knn_struct_size_matches_c():
    assert ctypes.sizeof(_lib.IpaKnnShape) == 4 * 8 + 4 + 4


def test_knn_validation_before_launch(lib):
    def ks(**kw):
        base = dict(B=2, N=300, k=20, nbins=20, dmax=20.0, dgram_dtype=0)
        base.update(kw)
        return _lib.IpaKnnShape(base["B"], base["N"], base["k"], base["nbins"], base["dmax"], base["dgram_dtype"])

    call = lambda s, t=4096, m=None, i=4096, d=4096, g=4096: lib.ipa_knn_distogram(ctypes.byref(s), t, m, i, d, g, None)
    assert lib.ipa_knn_distogram(None, 4096, None, 4096, None, None, None) == 1
    assert call(ks(), t=None) == 1
    assert call(ks(), i=None) == 1
    for bad in (dict(B=0), dict(N=0), dict(k=0), dict(k=65), dict(nbins=0), dict(nbins=5000), dict(dmax=0.0),
                dict(dmax=-1.0), dict(dmax=float("inf")), dict(dmax=float("nan")), dict(N=(1 << 30) + 1)):
        assert call(ks(**bad)) == 2, bad
    assert call(ks(dgram_dtype=5)) == 3
    assert call(ks(), t=4100) == 4
    assert call(ks(), m=4097) == 4
    assert call(ks(), i=4104) == 4
    assert call(ks(), d=4104) == 4
    assert call(ks(), g=4104) == 4


def test_backward_validation_before_launch(lib):
    s = _shape(dtype="f32")
    assert _lib.backward_workspace_bytes(s) > 0
    # bf16 inputs: the workspace also holds their fp32 copies
    assert _lib.backward_workspace_bytes(_shape(dtype="bf16")) > _lib.backward_workspace_bytes(s)
    bad_dt = _shape(dtype="f32")
    bad_dt.dtype = 7
    assert _lib.backward_workspace_bytes(bad_dt) == 0
    assert _lib.backward_workspace_bytes(_shape(dtype="f32", P=6)) == 0     # 3P > 16
    assert _lib.backward_workspace_bytes(_shape(dtype="f32", Cz=200)) == 0  # D + R Cz > 256
    assert _lib.backward_workspace_bytes(_shape(dtype="f32", N=0)) == 0
    # grows linearly with N (no N^2 array)
    w1 = _lib.backward_workspace_bytes(_shape(dtype="f32", B=1, N=8192))
    w2 = _lib.backward_workspace_bytes(_shape(dtype="f32", B=1, N=16384))
    assert 1.9 < w2 / w1 < 2.1
    fields = [n for n, _ in _lib.IpaLiftIn._fields_ if n != "pair_mask"]
    li = _lib.IpaLiftIn(**{n: 4096 for n in fields})
    ei = _lib.IpaEpiIn(4096, 4096, 4096, 4096, 4096)
    gr = _lib.IpaGrads(*[4096] * len(_lib.GRAD_KEYS))
    big = 1 << 40
    call = lambda s, li=li, ei=ei, gr=gr, du=4096, ws=4096, n=big: lib.ipa_backward(
        ctypes.byref(s), ctypes.byref(li), ctypes.byref(ei), du, 4096, ws, n, ctypes.byref(gr), None)
    assert call(s, du=None) == 1
    assert call(s, ws=None) == 1
    gr0 = _lib.IpaGrads(*[4096] * len(_lib.GRAD_KEYS))
    gr0.zr = None
    assert call(s, gr=gr0) == 1
    assert call(bad_dt) == 3
    assert call(_shape(dtype="f32", N=0)) == 2
    gr1 = _lib.IpaGrads(*[4096] * len(_lib.GRAD_KEYS))
    gr1.q = 4100
    assert call(s, gr=gr1) == 4
    assert call(s, n=16) == 2                                            # workspace too small


def test_bias_struct_size_matches_c():
    assert ctypes.sizeof(_lib.IpaBiasShape) == 7 * 8 + 4 * 4


def test_bias_attention_validation_before_launch(lib):
    def bs(**kw):
        base = dict(B=2, N=300, M=300, H=4, D=64, Dv=64, R=2, dtype=1, phi_dtype=0, causal=0, scale=0.125)
        base.update(kw)
        return _lib.IpaBiasShape(*[base[n] for n, _ in _lib.IpaBiasShape._fields_])

    ws = _lib.ipa_bias_workspace_bytes(bs())
    assert ws > 0
    # linear in the sequence lengths (no [N, M] array)
    w1 = _lib.ipa_bias_workspace_bytes(bs(N=8192, M=8192))
    w2 = _lib.ipa_bias_workspace_bytes(bs(N=16384, M=16384))
    assert 1.9 < w2 / w1 < 2.1
    for bad in (dict(B=0), dict(N=0), dict(M=0), dict(H=0), dict(D=0), dict(Dv=0), dict(R=-1),
                dict(scale=float("inf")), dict(scale=float("nan")), dict(causal=1, M=301), dict(H=70000)):
        assert _lib.ipa_bias_workspace_bytes(bs(**bad)) == 0, bad
    for unsup in (dict(dtype=3), dict(phi_dtype=2), dict(Dv=257), dict(D=250, R=3)):
        assert _lib.ipa_bias_workspace_bytes(bs(**unsup)) == 0, unsup
    assert _lib.ipa_bias_workspace_bytes(bs(D=247, R=3)) > 0          # D + 3R = 256
    assert _lib.ipa_bias_workspace_bytes(bs(R=0)) > 0

    big = 1 << 40
    def call(s, q=4096, k=4096, v=4096, pq=4096, pk=4096, km=None, o=4096, lse=4096, w=4096, n=big):
        return lib.ipa_bias_attention(ctypes.byref(s), q, k, v, pq, pk, km, o, lse, w, n, None)
    assert lib.ipa_bias_attention(None, 4096, 4096, 4096, 4096, 4096, None, 4096, 4096, 4096, big, None) == 1
    for name in ("q", "k", "v", "pq", "pk", "o", "lse", "w"):
        assert call(bs(), **{name: None}) == 1, name
    # factors are optional without a bias: the call gets past the pointer checks
    # (and stops at the misaligned q, before any launch)
    assert call(bs(R=0), q=4100, pq=None, pk=None) == 4
    assert call(bs(N=0)) == 2
    assert call(bs(causal=1, M=200)) == 2
    assert call(bs(dtype=5)) == 3
    assert call(bs(Dv=300)) == 3
    assert call(bs(), n=ws - 1) == 2                                  # workspace too small
    for name in ("q", "k", "v", "pq", "pk", "o", "lse", "w"):
        assert call(bs(), **{name: 4100}) == 4, name
    assert call(bs(), km=4097) == 4


def test_noalloc_rejects_shapes_beyond_its_scratch(lib):
    """ipa_forward_noalloc checks the shape against its static 128 MiB before
    any device call: N = 16384 (H = 8) needs ~280 MB."""
    s = _shape(B=1, N=16384)
    fields = [n for n, _ in _lib.IpaLiftIn._fields_ if n != "pair_mask"]
    li = _lib.IpaLiftIn(**{n: 4096 for n in fields})
    ei = _lib.IpaEpiIn(4096, 4096, 4096, 4096, 4096)
    assert lib.ipa_forward_noalloc(ctypes.byref(s), ctypes.byref(li), ctypes.byref(ei), 4096, 4096, None) == 7
    assert lib.ipa_forward_noalloc(ctypes.byref(s), ctypes.byref(li), ctypes.byref(ei), None, 4096, None) == 1
    li.q = 4100
    assert lib.ipa_forward_noalloc(ctypes.byref(_shape(B=1, N=100)), ctypes.byref(li), ctypes.byref(ei), 4096, 4096,
                                   None) == 4


def test_stacked_layout_shapes_and_validation(lib):
    """The stacked point-layout comparison: standard widths on the bf16 path
    only, a smaller lifted buffer (two geometric K-steps of 16 instead of
    three), the same validation as ipa_lift / ipa_flash_fwd."""
    s = _shape()
    std, stk = _lib.lifted_bytes(s, False), _lib.lifted_bytes(s, False, stacked=True)
    assert 0 < stk < std
    # the key rows lose 16 elements of 2 bytes per residue and head
    assert std - stk >= 2 * 8 * 320 * 16 * 2 - 4 * 256
    assert _lib.lifted_bytes(_shape(dtype="f32"), False, stacked=True) == 0
    assert _lib.lifted_bytes(_shape(P=3), False, stacked=True) == 0
    assert _lib.lifted_bytes(_shape(R=3), False, stacked=True) == 0
    assert _lib.lifted_bytes(_shape(Cz=32), False, stacked=True) == 0
    fields = [n for n, _ in _lib.IpaLiftIn._fields_ if n != "pair_mask"]
    li = _lib.IpaLiftIn(**{n: 4096 for n in fields})
    assert lib.ipa_lift_stacked(None, ctypes.byref(li), 4096, 1 << 40, None) == 1
    assert lib.ipa_lift_stacked(ctypes.byref(s), ctypes.byref(li), 4096, stk - 1, None) == 2
    li.k = 4100
    assert lib.ipa_lift_stacked(ctypes.byref(s), ctypes.byref(li), 4096, 1 << 40, None) == 4
    assert lib.ipa_lift_stacked(ctypes.byref(_shape(P=3)), ctypes.byref(li), 4096, 1 << 40, None) == 3
    assert lib.ipa_flash_fwd_stacked(ctypes.byref(s), None, 4096, 4096, None) == 1
    assert lib.ipa_flash_fwd_stacked(ctypes.byref(s), 4096, 4100, 4096, None) == 4
    assert lib.ipa_flash_fwd_stacked(ctypes.byref(_shape(dtype="f32")), 4096, 4096, 4096, None) == 3

