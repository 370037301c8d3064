"""ctypes binding of libflashipa.so (the C ABI in include/flashipa.h).

Argument marshalling only: every step of the forward runs in the library's
HIP kernels; torch provides device memory and the current stream.  There is
no fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# FLASHIPA_LIBRARY may name another build of the same library (same ABI)
LIB_PATH = os.environ.get("FLASHIPA_LIBRARY", os.path.join(HERE, "libflashipa.so"))

IPA_F32, IPA_BF16 = 0, 1
STATUS = {0: "IPA_OK", 1: "IPA_ERR_NULL", 2: "IPA_ERR_SHAPE", 3: "IPA_ERR_UNSUPPORTED",
          4: "IPA_ERR_ALIGN", 5: "IPA_ERR_LAUNCH", 6: "IPA_ERR_DEVICE", 7: "IPA_ERR_SCRATCH"}
EXPORTS = ("ipa_lifted_bytes", "ipa_o_width", "ipa_lift", "ipa_flash_fwd", "ipa_epilogue_workspace_bytes",
           "ipa_epilogue", "ipa_lifted_bytes_stacked", "ipa_lift_stacked", "ipa_flash_fwd_stacked",
           "ipa_logit_rows", "ipa_backward_workspace_bytes", "ipa_backward", "ipa_knn_distogram",
           "ipa_bias_workspace_bytes", "ipa_bias_attention", "ipa_forward_noalloc", "ipa_status_string",
           "ipa_version")
GRAD_KEYS = ("q", "k", "v", "q_points", "k_points", "v_points", "rotation", "translation",
             "point_weight_raw", "w_pair", "zl", "zr", "w_out", "b_out")


class IpaShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("B", "N", "H", "D", "Dv", "P", "Q", "Cz", "R", "Cout")] + \
               [("dtype", ctypes.c_int32), ("eps", ctypes.c_float)]


class IpaLiftIn(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("q", "k", "v", "q_points", "k_points", "v_points", "rotation",
                                                "translation", "point_weight_raw", "w_pair", "zl", "zr",
                                                "mask", "pair_mask")]


class IpaEpiIn(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("zl", "rotation", "translation", "w_out", "b_out")]


class IpaGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in GRAD_KEYS]


class IpaKnnShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("B", "N", "k", "nbins")] + \
               [("dmax", ctypes.c_float), ("dgram_dtype", ctypes.c_int32)]


class IpaBiasShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("B", "N", "M", "H", "D", "Dv", "R")] + \
               [("dtype", ctypes.c_int32), ("phi_dtype", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("scale", ctypes.c_float)]


class IPAError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} returned {STATUS.get(code, code)}")
        self.code = code


_LIB = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise ImportError(f"{path} not found: build it first (python -m rna_structure_amd.build)")
    lib = ctypes.CDLL(path)
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    sp = ctypes.POINTER(IpaShape)
    lib.ipa_lifted_bytes.argtypes = [sp, ctypes.c_int]
    lib.ipa_lifted_bytes.restype = sz
    lib.ipa_o_width.argtypes = [sp]
    lib.ipa_o_width.restype = i64
    lib.ipa_lift.argtypes = [sp, ctypes.POINTER(IpaLiftIn), vp, sz, vp]
    lib.ipa_lift.restype = ctypes.c_int
    lib.ipa_flash_fwd.argtypes = [sp, vp, vp, vp, vp]
    lib.ipa_flash_fwd.restype = ctypes.c_int
    lib.ipa_lifted_bytes_stacked.argtypes = [sp, ctypes.c_int]
    lib.ipa_lifted_bytes_stacked.restype = sz
    lib.ipa_lift_stacked.argtypes = [sp, ctypes.POINTER(IpaLiftIn), vp, sz, vp]
    lib.ipa_lift_stacked.restype = ctypes.c_int
    lib.ipa_flash_fwd_stacked.argtypes = [sp, vp, vp, vp, vp]
    lib.ipa_flash_fwd_stacked.restype = ctypes.c_int
    lib.ipa_epilogue_workspace_bytes.argtypes = [sp]
    lib.ipa_epilogue_workspace_bytes.restype = sz
    lib.ipa_epilogue.argtypes = [sp, vp, sz, vp, vp, ctypes.POINTER(IpaEpiIn), vp, vp, vp]
    lib.ipa_epilogue.restype = ctypes.c_int
    lib.ipa_logit_rows.argtypes = [sp, vp, i64, i64, i64, i64, vp, vp]
    lib.ipa_logit_rows.restype = ctypes.c_int
    lib.ipa_backward_workspace_bytes.argtypes = [sp]
    lib.ipa_backward_workspace_bytes.restype = sz
    lib.ipa_backward.argtypes = [sp, ctypes.POINTER(IpaLiftIn), ctypes.POINTER(IpaEpiIn), vp, vp, vp, sz,
                                 ctypes.POINTER(IpaGrads), vp]
    lib.ipa_backward.restype = ctypes.c_int
    lib.ipa_knn_distogram.argtypes = [ctypes.POINTER(IpaKnnShape), vp, vp, vp, vp, vp, vp]
    lib.ipa_knn_distogram.restype = ctypes.c_int
    lib.ipa_bias_workspace_bytes.argtypes = [ctypes.POINTER(IpaBiasShape)]
    lib.ipa_bias_workspace_bytes.restype = sz
    lib.ipa_bias_attention.argtypes = [ctypes.POINTER(IpaBiasShape), vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ipa_bias_attention.restype = ctypes.c_int
    lib.ipa_forward_noalloc.argtypes = [sp, ctypes.POINTER(IpaLiftIn), ctypes.POINTER(IpaEpiIn), vp, vp, vp]
    lib.ipa_forward_noalloc.restype = ctypes.c_int
    lib.ipa_status_string.argtypes = [ctypes.c_int]
    lib.ipa_status_string.restype = ctypes.c_char_p
    lib.ipa_version.argtypes = []
    lib.ipa_version.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def make_shape(shape, eps: float = 1e-8) -> IpaShape:
    """IpaShape from an object with B,N,H,D,Dv,P,Q,Cz,R,Cout and dtype ('f32'/'bf16')."""
    dt = {"f32": IPA_F32, "bf16": IPA_BF16}[shape.dtype]
    return IpaShape(shape.B, shape.N, shape.H, shape.D, shape.Dv, shape.P, shape.Q, shape.Cz, shape.R,
                    shape.Cout, dt, float(eps))


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check(fn, code):
    if code != 0:
        raise IPAError(fn, code)


def lifted_bytes(s: IpaShape, with_pair_mask: bool, stacked: bool = False) -> int:
    fn = load().ipa_lifted_bytes_stacked if stacked else load().ipa_lifted_bytes
    return int(fn(ctypes.byref(s), int(bool(with_pair_mask))))


def o_width(s: IpaShape) -> int:
    return int(load().ipa_o_width(ctypes.byref(s)))


def ipa_lift(s: IpaShape, t: dict, lifted, stream=None, stacked: bool = False):
    lib = load()
    li = IpaLiftIn(*[_ptr(t.get(n)) for n in ("q", "k", "v", "q_points", "k_points", "v_points", "rotation",
                                              "translation", "point_weight_raw", "w_pair", "zl", "zr",
                                              "mask", "pair_mask")])
    name = "ipa_lift_stacked" if stacked else "ipa_lift"
    _check(name, getattr(lib, name)(ctypes.byref(s), ctypes.byref(li), _ptr(lifted), lifted.numel() *
                                    lifted.element_size(), _stream(stream)))


def ipa_flash_fwd(s: IpaShape, lifted, o, lse, stream=None, stacked: bool = False):
    name = "ipa_flash_fwd_stacked" if stacked else "ipa_flash_fwd"
    _check(name, getattr(load(), name)(ctypes.byref(s), _ptr(lifted), _ptr(o), _ptr(lse), _stream(stream)))


def epilogue_workspace_bytes(s: IpaShape) -> int:
    return int(load().ipa_epilogue_workspace_bytes(ctypes.byref(s)))


def ipa_epilogue(s: IpaShape, workspace, o, lse, t: dict, update, local_points, stream=None):
    ei = IpaEpiIn(*[_ptr(t[n]) for n in ("zl", "rotation", "translation", "w_out", "b_out")])
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("ipa_epilogue", load().ipa_epilogue(ctypes.byref(s), _ptr(workspace), nbytes, _ptr(o), _ptr(lse),
                                               ctypes.byref(ei), _ptr(update), _ptr(local_points), _stream(stream)))


def ipa_forward_noalloc(s: IpaShape, t: dict, update, local_points, stream=None):
    """The whole forward in one call that allocates nothing (static scratch)."""
    li = IpaLiftIn(*[_ptr(t.get(n)) for n in ("q", "k", "v", "q_points", "k_points", "v_points", "rotation",
                                              "translation", "point_weight_raw", "w_pair", "zl", "zr",
                                              "mask", "pair_mask")])
    ei = IpaEpiIn(*[_ptr(t[n]) for n in ("zl", "rotation", "translation", "w_out", "b_out")])
    _check("ipa_forward_noalloc", load().ipa_forward_noalloc(ctypes.byref(s), ctypes.byref(li), ctypes.byref(ei),
                                                             _ptr(update), _ptr(local_points), _stream(stream)))


def ipa_logit_rows(s: IpaShape, lifted, b: int, h: int, row0: int, nrows: int, out, stream=None):
    _check("ipa_logit_rows", load().ipa_logit_rows(ctypes.byref(s), _ptr(lifted), b, h, row0, nrows,
                                                   _ptr(out), _stream(stream)))


def ipa_knn_distogram(s: IpaKnnShape, translation, mask, nn_index, nn_dist=None, dgram=None, stream=None):
    _check("ipa_knn_distogram", load().ipa_knn_distogram(ctypes.byref(s), _ptr(translation), _ptr(mask),
                                                         _ptr(nn_index), _ptr(nn_dist), _ptr(dgram),
                                                         _stream(stream)))


def backward_workspace_bytes(s: IpaShape) -> int:
    return int(load().ipa_backward_workspace_bytes(ctypes.byref(s)))


def ipa_backward(s: IpaShape, t: dict, d_update, d_local, workspace, grads: dict, stream=None):
    lib = load()
    li = IpaLiftIn(*[_ptr(t.get(n)) for n in ("q", "k", "v", "q_points", "k_points", "v_points", "rotation",
                                              "translation", "point_weight_raw", "w_pair", "zl", "zr",
                                              "mask", "pair_mask")])
    ei = IpaEpiIn(*[_ptr(t[n]) for n in ("zl", "rotation", "translation", "w_out", "b_out")])
    gr = IpaGrads(*[_ptr(grads[n]) for n in GRAD_KEYS])
    _check("ipa_backward", lib.ipa_backward(ctypes.byref(s), ctypes.byref(li), ctypes.byref(ei), _ptr(d_update),
                                            _ptr(d_local), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                            ctypes.byref(gr), _stream(stream)))


class IPABackward:
    """Workspace, gradient buffers and the backward call for a fixed shape.

    t are device inputs in the shape's dtype (device_inputs); gradients are
    fp32, each shaped like its input, and rewritten by every call."""

    def __init__(self, shape, eps: float = 1e-8, device="cuda"):
        import torch
        load()
        self.shape = shape
        self.s = make_shape(shape, eps)
        nbytes = backward_workspace_bytes(self.s)
        if nbytes == 0:
            raise IPAError("ipa_backward_workspace_bytes", 3)
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.grads = None

    def __call__(self, t: dict, d_update, d_local, stream=None) -> dict:
        import torch
        if self.grads is None:
            self.grads = {n: torch.empty_like(t[n], dtype=torch.float32) for n in GRAD_KEYS}
        ipa_backward(self.s, t, d_update, d_local, self.ws, self.grads, stream)
        return self.grads


class KnnDistogram:
    """Output buffers and the call of the kNN distogram for a fixed shape.

    translation [B,N,3] fp32 and mask [B,N] uint8 (or None) are device tensors;
    nn_index [B,N,k] int32, nn_dist [B,N,k] fp32 and dgram [B,N,k,nbins]
    (fp32 or bf16) are allocated here and rewritten by every call."""

    def __init__(self, B: int, N: int, k: int = 20, nbins: int = 20, dmax: float = 20.0,
                 dgram_dtype: str = "f32", with_dist: bool = True, with_dgram: bool = True, device="cuda"):
        import torch
        load()
        dt = {"f32": IPA_F32, "bf16": IPA_BF16}[dgram_dtype]
        self.s = IpaKnnShape(B, N, k, nbins, float(dmax), dt)
        self.nn_index = torch.empty(B, N, k, dtype=torch.int32, device=device)
        self.nn_dist = torch.empty(B, N, k, dtype=torch.float32, device=device) if with_dist else None
        tdt = torch.bfloat16 if dgram_dtype == "bf16" else torch.float32
        self.dgram = torch.empty(B, N, k, nbins, dtype=tdt, device=device) if with_dgram else None

    def __call__(self, translation, mask=None, stream=None) -> dict:
        ipa_knn_distogram(self.s, translation, mask, self.nn_index, self.nn_dist, self.dgram, stream)
        return dict(index=self.nn_index, dist=self.nn_dist, dgram=self.dgram)


def ipa_bias_workspace_bytes(s: IpaBiasShape) -> int:
    return int(load().ipa_bias_workspace_bytes(ctypes.byref(s)))


def ipa_bias_attention(s: IpaBiasShape, q, k, v, phi_q, phi_k, key_mask, o, lse, workspace, stream=None):
    _check("ipa_bias_attention", load().ipa_bias_attention(
        ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(phi_q), _ptr(phi_k), _ptr(key_mask), _ptr(o), _ptr(lse),
        _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(stream)))


class BiasAttention:
    """Workspace, output buffers and the call of attention with a low-rank
    bias for a fixed shape.  q [B,N,H,D], k [B,M,H,D], v [B,M,H,Dv],
    (device tensors in `dtype`), phi_q [B,N,H,R], phi_k [B,M,H,R] (in
    `phi_dtype`) and key_mask [B,M] uint8 (or None); o [B,N,H,Dv] and
    lse [B,H,N] (fp32) are allocated here and rewritten by every call."""

    def __init__(self, B: int, N: int, M: int, H: int, D: int, Dv: int, R: int, scale: float,
                 causal: bool = False, dtype: str = "bf16", phi_dtype: str = "f32", device="cuda"):
        import torch
        load()
        dts = {"f32": IPA_F32, "bf16": IPA_BF16}
        self.s = IpaBiasShape(B, N, M, H, D, Dv, R, dts[dtype], dts[phi_dtype], int(bool(causal)), float(scale))
        nbytes = ipa_bias_workspace_bytes(self.s)
        if nbytes == 0:
            raise IPAError("ipa_bias_workspace_bytes", 3)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.o = torch.empty(B, N, H, Dv, dtype=torch.float32, device=device)
        self.lse = torch.empty(B, H, N, dtype=torch.float32, device=device)

    def __call__(self, q, k, v, phi_q=None, phi_k=None, key_mask=None, stream=None) -> dict:
        ipa_bias_attention(self.s, q, k, v, phi_q, phi_k, key_mask, self.o, self.lse, self.workspace, stream)
        return dict(o=self.o, lse=self.lse)


_FLOAT_KEYS = ("q", "k", "v", "q_points", "k_points", "v_points", "rotation", "translation",
               "point_weight_raw", "w_pair", "zl", "zr", "w_out", "b_out")


def device_inputs(inp: dict, device="cuda") -> dict:
    """Copy a host input set (numpy arrays) to device tensors of the run dtype."""
    import torch
    dt = torch.bfloat16 if inp["shape"].dtype == "bf16" else torch.float32
    out = {}
    for key in _FLOAT_KEYS:
        a = np.ascontiguousarray(inp[key], dtype=np.float32)
        out[key] = torch.from_numpy(a).to(device=device).to(dt).contiguous()
    out["mask"] = torch.from_numpy(np.ascontiguousarray(inp["mask"]).astype(np.uint8)).to(device)
    pm = inp.get("pair_mask")
    out["pair_mask"] = None if pm is None else torch.from_numpy(np.ascontiguousarray(pm).astype(np.uint8)).to(device)
    return out


class FlashIPA:
    """Buffers and the three calls of one forward for a fixed problem shape.
    stacked=True runs the lift and the fused attention with the pages' stacked
    point layout (ipa_lift_stacked / ipa_flash_fwd_stacked, a comparison)."""

    def __init__(self, shape, eps: float = 1e-8, with_pair_mask: bool = False, device="cuda", stacked: bool = False):
        import torch
        load()
        self.shape = shape
        self.stacked = stacked
        self.s = make_shape(shape, eps)
        nbytes = lifted_bytes(self.s, with_pair_mask, stacked)
        if nbytes == 0:
            raise IPAError("ipa_lifted_bytes_stacked" if stacked else "ipa_lifted_bytes", 3)
        self.lifted = torch.empty(nbytes, dtype=torch.uint8, device=device)
        ebytes = epilogue_workspace_bytes(self.s)
        if ebytes == 0:
            raise IPAError("ipa_epilogue_workspace_bytes", 3)
        self.epi_ws = torch.empty(ebytes, dtype=torch.uint8, device=device)
        B, N, H, Q = shape.B, shape.N, shape.H, shape.Q
        self.o = torch.empty(B, N, H, o_width(self.s), dtype=torch.float32, device=device)
        self.lse = torch.empty(B, H, N, dtype=torch.float32, device=device)
        self.update = torch.empty(B, N, shape.Cout, dtype=torch.float32, device=device)
        self.local_points = torch.empty(B, N, H, Q, 3, dtype=torch.float32, device=device)

    def poison(self):
        """Fill the workspace with 0xFF bytes and the outputs with NaN (for
        tests: whatever a kernel fails to write, or reads before it is
        written, then shows up)."""
        self.lifted.fill_(255)
        self.epi_ws.fill_(255)
        for buf in (self.o, self.lse, self.update, self.local_points):
            buf.fill_(float("nan"))

    def lift(self, t: dict, stream=None):
        ipa_lift(self.s, t, self.lifted, stream, self.stacked)

    def attend(self, stream=None):
        ipa_flash_fwd(self.s, self.lifted, self.o, self.lse, stream, self.stacked)

    def epilogue(self, t: dict, stream=None):
        ipa_epilogue(self.s, self.epi_ws, self.o, self.lse, t, self.update, self.local_points, stream)

    def forward(self, t: dict, stream=None):
        self.lift(t, stream)
        self.attend(stream)
        self.epilogue(t, stream)
        return dict(update=self.update, local_points=self.local_points, o=self.o, lse=self.lse)

    def logit_rows(self, b: int, h: int, row0: int, nrows: int, stream=None):
        import torch
        if self.stacked:
            raise ValueError("ipa_logit_rows reads the standard layout only")
        out = torch.empty(nrows, self.shape.N, dtype=torch.float32, device=self.o.device)
        ipa_logit_rows(self.s, self.lifted, b, h, row0, nrows, out, stream)
        return out


def forward(inp_dev: dict, shape, eps: float = 1e-8) -> dict:
    """One forward on device tensors (see device_inputs)."""
    f = FlashIPA(shape, eps, with_pair_mask=inp_dev.get("pair_mask") is not None,
                 device=inp_dev["q"].device)
    return f.forward(inp_dev)
