"""Python binding of libqlora: the gfx950 QLoRA adapted linear.

Argument marshalling only.  Every step of the layer runs in the HIP kernels
of ``libqlora.so`` (built in-tree by ``parameter_efficient_fine_nf4_amd/build.py``);
torch provides device memory and the current stream.  Importing this module
fails loudly when the library has not been built.

The calls mirror include/qlora.h:

* ``quantize(W0)``                     -> ``NF4Weight``
* ``forward(X, w, A, B, alpha)``       -> ``Y`` (and ``T_save``)
* ``backward(dY, X, w, A, B, alpha)``  -> ``dX, dA, dB``
* ``merge(w, A, B, alpha)``            -> bf16 ``W``
* ``unmerge(W, A, B, alpha)``          -> bf16 ``W0``
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# QLORA_LIB_PATH selects another build of the same library (the host-side
# sanitizer build that build.py --sanitize writes under _build/).
LIB_PATH = os.environ.get("QLORA_LIB_PATH") or os.path.join(_HERE, "libqlora.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with "
        "`python parameter_efficient_fine_nf4_amd/build.py` (hipcc, gfx950)")

_lib = ctypes.CDLL(LIB_PATH)

_i64, _i32, _f32, _sz, _vp = (ctypes.c_int64, ctypes.c_int32, ctypes.c_float,
                              ctypes.c_size_t, ctypes.c_void_p)


class _Nf4Desc(ctypes.Structure):
    _fields_ = [("d", _i64), ("k", _i64), ("codes", _vp), ("absmax_q", _vp),
                ("absmax_scale", _vp), ("absmax_mean", _vp)]


_P = ctypes.POINTER(_Nf4Desc)
_sigs = {
    "qlora_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "qlora_version": (ctypes.c_int, []),
    "qlora_nf4_levels": (ctypes.c_int, [ctypes.POINTER(ctypes.c_float)]),
    "qlora_nf4_sizes": (ctypes.c_int, [_i64, _i64, ctypes.POINTER(_sz), ctypes.POINTER(_sz),
                                       ctypes.POINTER(_sz), ctypes.POINTER(_sz)]),
    "qlora_quantize_workspace_bytes": (_sz, [_i64, _i64]),
    "nf4_quantize": (ctypes.c_int, [_vp, _i64, _i64, _P, _vp, _sz, _vp]),
    "qlora_tsave_bytes": (_sz, [_i64, _i32]),
    "qlora_forward_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32]),
    "qlora_forward": (ctypes.c_int, [_vp, _i64, _P, _vp, _vp, _i32, _f32, _vp, _vp, _vp, _sz, _vp]),
    "qlora_backward_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32]),
    "qlora_backward": (ctypes.c_int, [_vp, _vp, _i64, _P, _vp, _vp, _i32, _f32, _vp, _vp, _vp,
                                      _vp, _vp, _sz, _vp]),
    "qlora_backward_noalloc": (ctypes.c_int, [_vp, _vp, _i64, _P, _vp, _vp, _i32, _f32, _vp, _vp, _vp,
                                              _vp, _vp]),
    "qlora_forward_sections": (ctypes.c_int, [_vp, _i64, _P, _i32, _vp, _vp, _i32, _f32, _vp, _vp, _vp,
                                              _sz, _vp]),
    "qlora_backward_sections": (ctypes.c_int, [_vp, _vp, _i64, _P, _i32, _vp, _vp, _i32, _f32, _vp,
                                               _vp, _vp, _vp, _vp, _sz, _vp]),
    "qlora_forward_dropout_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32]),
    "qlora_backward_dropout_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32]),
    "qlora_forward_dropout": (ctypes.c_int, [_vp, _i64, _P, _vp, _vp, _i32, _f32, _vp, _f32, _vp, _vp, _vp,
                                             _vp, _sz, _vp]),
    "qlora_backward_dropout": (ctypes.c_int, [_vp, _vp, _i64, _P, _vp, _vp, _i32, _f32, _vp, _f32, _vp, _vp,
                                              _vp, _vp, _vp, _vp, _sz, _vp]),
    "qlora_forward_multi_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32, _i32]),
    "qlora_forward_multi": (ctypes.c_int, [_vp, _i64, _P, _i32, _vp, _vp, _vp, _i32, _f32, _vp, _vp,
                                           _sz, _vp]),
    "qlora_adam_step": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _f32, _f32, _f32, _f32, _f32, _i64, _vp]),
    "lora_merge": (ctypes.c_int, [_P, _vp, _vp, _i32, _f32, _vp, _vp]),
    "lora_unmerge": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _i32, _f32, _vp, _vp]),
    "qlora_timing_enable": (ctypes.c_int, [ctypes.c_int]),
    "qlora_timing_collect": (ctypes.c_int, []),
    "qlora_timing_query": (ctypes.c_int, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                          ctypes.POINTER(_i64)]),
    "qlora_timing_reset": (ctypes.c_int, []),
}
for _name, (_res, _args) in _sigs.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_sigs)
STATUS = {0: "QLORA_OK", 1: "QLORA_ERR_NULL", 2: "QLORA_ERR_SHAPE", 3: "QLORA_ERR_RANK",
          4: "QLORA_ERR_ALIGN", 5: "QLORA_ERR_WORKSPACE", 6: "QLORA_ERR_ALPHA",
          7: "QLORA_ERR_ALIAS", 8: "QLORA_ERR_HIP"}


class QloraError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        msg = _lib.qlora_status_string(status).decode()
        super().__init__(f"{call} failed: {STATUS.get(status, status)} ({msg})")


def _check(status: int, call: str) -> None:
    if status != 0:
        raise QloraError(status, call)


def lib() -> ctypes.CDLL:
    """The loaded ctypes library (raw C ABI)."""
    return _lib


def nf4_levels() -> list:
    """The library's 16 NF4 levels (host computation)."""
    buf = (ctypes.c_float * 16)()
    _check(_lib.qlora_nf4_levels(buf), "qlora_nf4_levels")
    return list(buf)


def nf4_sizes(d: int, k: int) -> dict:
    out = [_sz() for _ in range(4)]
    _check(_lib.qlora_nf4_sizes(d, k, *[ctypes.byref(o) for o in out]), "qlora_nf4_sizes")
    return dict(zip(("codes", "absmax_q", "absmax_scale", "absmax_mean"), (o.value for o in out)))


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    """Raw handle of the current stream of ``device`` (torch's C accessor:
    a few microseconds cheaper per call than building a Stream object)."""
    idx = device.index if device.index is not None else torch.cuda.current_device()
    return torch._C._cuda_getCurrentRawStream(idx)


def _workspace(nbytes: int, device) -> torch.Tensor | None:
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


@dataclass
class NF4Weight:
    """Device buffers of one NF4-quantised d x k weight (caller-owned).

    With ``nsec`` > 1 the rows stack nsec weights of d/nsec rows each,
    quantised one by one (see ``quantize_sections``), and ``absmax_mean``
    holds their nsec means."""
    d: int
    k: int
    codes: torch.Tensor         # uint8 [d*k/2]
    absmax_q: torch.Tensor      # uint8 [d*k/64]   (FP8 E4M3FN)
    absmax_scale: torch.Tensor  # float32 [ceil(n_b/256)]
    absmax_mean: torch.Tensor   # float32 [nsec]
    nsec: int = 1

    @staticmethod
    def empty(d: int, k: int, device, nsec: int = 1) -> "NF4Weight":
        sz = nf4_sizes(d, k)
        return NF4Weight(d, k,
                         torch.empty(sz["codes"], dtype=torch.uint8, device=device),
                         torch.empty(sz["absmax_q"], dtype=torch.uint8, device=device),
                         torch.empty(sz["absmax_scale"] // 4, dtype=torch.float32, device=device),
                         torch.empty(nsec, dtype=torch.float32, device=device), nsec)

    def section(self, p: int) -> "NF4Weight":
        """Section p as a single-weight view of the same buffers (its rows
        are whole second-level groups, so every array slices cleanly)."""
        ds = self.d // self.nsec
        nb = ds * self.k // 64
        assert self.nsec == 1 or nb % 256 == 0
        return NF4Weight(ds, self.k, self.codes[p * ds * self.k // 2:(p + 1) * ds * self.k // 2],
                         self.absmax_q[p * nb:(p + 1) * nb],
                         self.absmax_scale[p * (nb // 256):(p + 1) * (nb // 256)] if self.nsec > 1
                         else self.absmax_scale,
                         self.absmax_mean[p:p + 1])

    def desc(self) -> _Nf4Desc:
        return _Nf4Desc(self.d, self.k, self.codes.data_ptr(), self.absmax_q.data_ptr(),
                        self.absmax_scale.data_ptr(), self.absmax_mean.data_ptr())

    @property
    def device(self):
        return self.codes.device


def quantize(W0: torch.Tensor, out: NF4Weight | None = None) -> NF4Weight:
    """NF4 + double-quantised absmax of a d x k fp32 device tensor."""
    assert W0.dtype == torch.float32 and W0.dim() == 2 and W0.is_contiguous()
    d, k = W0.shape
    w = out if out is not None else NF4Weight.empty(d, k, W0.device)
    ws = _workspace(_lib.qlora_quantize_workspace_bytes(d, k), W0.device)
    desc = w.desc()
    _check(_lib.nf4_quantize(W0.data_ptr(), d, k, ctypes.byref(desc), _ptr(ws),
                             0 if ws is None else ws.numel(), _stream(W0.device)), "nf4_quantize")
    return w


def quantize_sections(W0s) -> NF4Weight:
    """Row-stacked NF4 storage of several d_p x k fp32 weights of one shape
    (e.g. a layer's q, k and v projections), each quantised on its own."""
    n = len(W0s)
    d, k = W0s[0].shape
    assert all(W.shape == (d, k) for W in W0s)
    w = NF4Weight.empty(n * d, k, W0s[0].device, nsec=n)
    for p, W in enumerate(W0s):
        quantize(W, out=w.section(p))
    return w


def _rank(A):
    return 0 if A is None else int(A.shape[0])


def forward(X: torch.Tensor, w: NF4Weight, A=None, B=None, alpha: float = 0.0,
            save_t: bool = False, out: torch.Tensor | None = None):
    """Y = X w~^T + (alpha/r) (X A^T) B^T (bf16).  With ``save_t`` also
    returns the saved T^T buffer for ``backward``."""
    assert w.nsec == 1, "a weight with row sections goes through forward_sections"
    M = X.shape[0]
    r = _rank(A)
    dev = X.device
    Y = out if out is not None else torch.empty((M, w.d), dtype=torch.bfloat16, device=dev)
    T = None
    if save_t and r > 0:
        T = torch.empty(max(1, _lib.qlora_tsave_bytes(M, r) // 2), dtype=torch.bfloat16, device=dev)
    ws = _workspace(_lib.qlora_forward_workspace_bytes(M, w.d, w.k, r), dev)
    desc = w.desc()
    _check(_lib.qlora_forward(X.data_ptr(), M, ctypes.byref(desc), _ptr(A), _ptr(B), r,
                              float(alpha), Y.data_ptr(), _ptr(T), _ptr(ws),
                              0 if ws is None else ws.numel(), _stream(dev)), "qlora_forward")
    return (Y, T) if save_t else Y


def backward(dY: torch.Tensor, X: torch.Tensor, w: NF4Weight, A=None, B=None,
             alpha: float = 0.0, T_saved=None, need_dx: bool = True):
    """(dX, dA, dB) of the adapted linear; dX is None when ``need_dx`` is
    False; dA/dB are None when r == 0."""
    assert w.nsec == 1, "a weight with row sections goes through backward_sections"
    M = X.shape[0]
    r = _rank(A)
    dev = X.device
    dX = torch.empty((M, w.k), dtype=torch.bfloat16, device=dev) if need_dx else None
    dA = torch.empty((r, w.k), dtype=torch.bfloat16, device=dev) if r else None
    dB = torch.empty((w.d, r), dtype=torch.bfloat16, device=dev) if r else None
    ws = _workspace(_lib.qlora_backward_workspace_bytes(M, w.d, w.k, r), dev)
    desc = w.desc()
    _check(_lib.qlora_backward(dY.data_ptr(), X.data_ptr(), M, ctypes.byref(desc), _ptr(A),
                               _ptr(B), r, float(alpha), _ptr(T_saved), _ptr(dX), _ptr(dA),
                               _ptr(dB), _ptr(ws), 0 if ws is None else ws.numel(),
                               _stream(dev)), "qlora_backward")
    return dX, dA, dB


def backward_noalloc(dY: torch.Tensor, X: torch.Tensor, w: NF4Weight, A=None, B=None,
                     alpha: float = 0.0, T_saved=None, out=None):
    """``backward`` through qlora_backward_noalloc: no workspace; the library
    uses its static per-GPU scratch array.  ``out`` = (dX, dA, dB) to write
    into preallocated tensors (dX may be None to skip it)."""
    assert w.nsec == 1
    M = X.shape[0]
    r = _rank(A)
    dev = X.device
    if out is None:
        out = (torch.empty((M, w.k), dtype=torch.bfloat16, device=dev),
               torch.empty((r, w.k), dtype=torch.bfloat16, device=dev) if r else None,
               torch.empty((w.d, r), dtype=torch.bfloat16, device=dev) if r else None)
    dX, dA, dB = out
    desc = w.desc()
    _check(_lib.qlora_backward_noalloc(dY.data_ptr(), X.data_ptr(), M, ctypes.byref(desc), _ptr(A),
                                       _ptr(B), r, float(alpha), _ptr(T_saved), _ptr(dX), _ptr(dA),
                                       _ptr(dB), _stream(dev)), "qlora_backward_noalloc")
    return dX, dA, dB


def forward_sections(X: torch.Tensor, w: NF4Weight, A=None, B=None, alpha: float = 0.0,
                     save_t: bool = False, out: torch.Tensor | None = None):
    """Y (M x d) of the w.nsec projections stacked in ``w`` that share the
    input X: section p's columns are X w~_p^T + (alpha/r) (X A_p^T) B_p^T,
    with A = [A_0; A_1; ...] ((nsec*r) x k) and B = [B_0; B_1; ...] (d x r)."""
    M = X.shape[0]
    rt = _rank(A)
    r = rt // w.nsec
    dev = X.device
    Y = out if out is not None else torch.empty((M, w.d), dtype=torch.bfloat16, device=dev)
    T = None
    if save_t and r > 0:
        T = torch.empty(max(1, _lib.qlora_tsave_bytes(M, rt) // 2), dtype=torch.bfloat16, device=dev)
    ws = _workspace(_lib.qlora_forward_workspace_bytes(M, w.d, w.k, rt), dev)
    desc = w.desc()
    _check(_lib.qlora_forward_sections(X.data_ptr(), M, ctypes.byref(desc), w.nsec, _ptr(A), _ptr(B),
                                       r, float(alpha), Y.data_ptr(), _ptr(T), _ptr(ws),
                                       0 if ws is None else ws.numel(), _stream(dev)),
           "qlora_forward_sections")
    return (Y, T) if save_t else Y


def forward_dropout(X: torch.Tensor, w: NF4Weight, A, B, alpha: float, keep: torch.Tensor, p: float,
                    save_t: bool = False, out: torch.Tensor | None = None, xd_out: torch.Tensor | None = None):
    """``forward`` with LoRA dropout on the adapter path's input: keep is an
    M x k uint8 mask (nonzero = kept), p the dropout probability.  With
    ``xd_out`` (M x k bf16) the dropped input is kept there for
    ``backward_dropout(..., Xd_saved=xd_out)``."""
    assert w.nsec == 1 and keep.dtype == torch.uint8 and keep.is_contiguous()
    M = X.shape[0]
    r = _rank(A)
    dev = X.device
    Y = out if out is not None else torch.empty((M, w.d), dtype=torch.bfloat16, device=dev)
    T = None
    if save_t and r > 0:
        T = torch.empty(max(1, _lib.qlora_tsave_bytes(M, r) // 2), dtype=torch.bfloat16, device=dev)
    ws = _workspace(_lib.qlora_forward_dropout_workspace_bytes(M, w.d, w.k, r), dev)
    desc = w.desc()
    _check(_lib.qlora_forward_dropout(X.data_ptr(), M, ctypes.byref(desc), _ptr(A), _ptr(B), r, float(alpha),
                                      keep.data_ptr(), float(p), Y.data_ptr(), _ptr(T), _ptr(xd_out), _ptr(ws),
                                      0 if ws is None else ws.numel(), _stream(dev)), "qlora_forward_dropout")
    return (Y, T) if save_t else Y


def backward_dropout(dY: torch.Tensor, X: torch.Tensor, w: NF4Weight, A, B, alpha: float,
                     keep: torch.Tensor, p: float, T_saved=None, need_dx: bool = True, Xd_saved=None):
    """``backward`` for ``forward_dropout`` (the same mask and p)."""
    assert w.nsec == 1 and keep.dtype == torch.uint8 and keep.is_contiguous()
    M = X.shape[0]
    r = _rank(A)
    dev = X.device
    dX = torch.empty((M, w.k), dtype=torch.bfloat16, device=dev) if need_dx else None
    dA = torch.empty((r, w.k), dtype=torch.bfloat16, device=dev) if r else None
    dB = torch.empty((w.d, r), dtype=torch.bfloat16, device=dev) if r else None
    ws = _workspace(_lib.qlora_backward_dropout_workspace_bytes(M, w.d, w.k, r), dev)
    desc = w.desc()
    _check(_lib.qlora_backward_dropout(dY.data_ptr(), X.data_ptr(), M, ctypes.byref(desc), _ptr(A), _ptr(B), r,
                                       float(alpha), keep.data_ptr(), float(p), _ptr(T_saved), _ptr(Xd_saved),
                                       _ptr(dX),
                                       _ptr(dA), _ptr(dB), _ptr(ws), 0 if ws is None else ws.numel(),
                                       _stream(dev)), "qlora_backward_dropout")
    return dX, dA, dB


def forward_multi(X: torch.Tensor, w: NF4Weight, A, B, idx: torch.Tensor, alpha: float,
                  out: torch.Tensor | None = None):
    """Y (M x d) with a per-token adapter: token m adds (alpha/r) (X[m]
    A_a^T) B_a^T for a = idx[m] in [0, nad), nothing otherwise.  A is
    (nad*r) x k, B is (nad*d) x r (blocks B_0, B_1, ...), idx int32 [M]."""
    assert w.nsec == 1 and idx.dtype == torch.int32 and idx.is_contiguous()
    M = X.shape[0]
    nad = B.shape[0] // w.d
    r = A.shape[0] // nad
    dev = X.device
    Y = out if out is not None else torch.empty((M, w.d), dtype=torch.bfloat16, device=dev)
    ws = _workspace(_lib.qlora_forward_multi_workspace_bytes(M, w.d, w.k, nad, r), dev)
    desc = w.desc()
    _check(_lib.qlora_forward_multi(X.data_ptr(), M, ctypes.byref(desc), nad, A.data_ptr(), B.data_ptr(),
                                    idx.data_ptr(), r, float(alpha), Y.data_ptr(), _ptr(ws),
                                    0 if ws is None else ws.numel(), _stream(dev)), "qlora_forward_multi")
    return Y


def backward_sections(dY: torch.Tensor, X: torch.Tensor, w: NF4Weight, A=None, B=None,
                      alpha: float = 0.0, T_saved=None, need_dx: bool = True):
    """(dX, dA, dB) for ``forward_sections``: dA stacks the sections' dA_p
    like A, dB their dB_p like B."""
    M = X.shape[0]
    rt = _rank(A)
    r = rt // w.nsec
    dev = X.device
    dX = torch.empty((M, w.k), dtype=torch.bfloat16, device=dev) if need_dx else None
    dA = torch.empty((rt, w.k), dtype=torch.bfloat16, device=dev) if rt else None
    dB = torch.empty((w.d, r), dtype=torch.bfloat16, device=dev) if rt else None
    ws = _workspace(_lib.qlora_backward_workspace_bytes(M, w.d, w.k, rt), dev)
    desc = w.desc()
    _check(_lib.qlora_backward_sections(dY.data_ptr(), X.data_ptr(), M, ctypes.byref(desc), w.nsec,
                                        _ptr(A), _ptr(B), r, float(alpha), _ptr(T_saved), _ptr(dX),
                                        _ptr(dA), _ptr(dB), _ptr(ws), 0 if ws is None else ws.numel(),
                                        _stream(dev)), "qlora_backward_sections")
    return dX, dA, dB


def adam_step(P: torch.Tensor, W: torch.Tensor, G: torch.Tensor, m: torch.Tensor, v: torch.Tensor,
              lr: float, step: int, beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8,
              weight_decay: float = 0.0) -> None:
    """One Adam step: W, m, v (fp32) in place, P = bf16(W); G bf16 gradients."""
    n = P.numel()
    assert P.dtype == torch.bfloat16 and G.dtype == torch.bfloat16 and G.numel() == n
    assert W.dtype == m.dtype == v.dtype == torch.float32 and W.numel() == m.numel() == v.numel() == n
    _check(_lib.qlora_adam_step(P.data_ptr(), W.data_ptr(), G.data_ptr(), m.data_ptr(), v.data_ptr(), n,
                                float(lr), float(beta1), float(beta2), float(eps), float(weight_decay),
                                int(step), _stream(P.device)), "qlora_adam_step")


def merge(w: NF4Weight, A=None, B=None, alpha: float = 0.0, out=None) -> torch.Tensor:
    """W = bf16(w~ + (alpha/r) B A), d x k bf16 (one section at a time:
    ``merge(w.section(p), A_p, B_p, alpha)``)."""
    assert w.nsec == 1, "merge the sections one at a time through NF4Weight.section"
    r = _rank(A)
    W = out if out is not None else torch.empty((w.d, w.k), dtype=torch.bfloat16, device=w.device)
    desc = w.desc()
    _check(_lib.lora_merge(ctypes.byref(desc), _ptr(A), _ptr(B), r, float(alpha), W.data_ptr(),
                           _stream(w.device)), "lora_merge")
    return W


def unmerge(W: torch.Tensor, A=None, B=None, alpha: float = 0.0, out=None) -> torch.Tensor:
    """W0 = bf16(W - (alpha/r) B A); ``out`` may be ``W`` itself."""
    r = _rank(A)
    d, k = W.shape
    O = out if out is not None else torch.empty_like(W)
    _check(_lib.lora_unmerge(W.data_ptr(), d, k, _ptr(A), _ptr(B), r, float(alpha), O.data_ptr(),
                             _stream(W.device)), "lora_unmerge")
    return O


class kernel_timing:
    """Context manager: per-kernel HIP-event timing of every launch made by
    the library inside the block.  ``totals()`` -> {name: (total_ms, n)}."""

    NAMES = ("quant_blocks", "quant_group_sums", "quant_mean", "quant_dq", "merge", "unmerge",
             "prep_adapters", "lora_proj", "lora_proj_finish", "token_reduce",
             "token_reduce_finish", "fwd_decode", "fwd_decode_finish", "fwd_rich", "dx", "drop_input", "adam",
             "fwd_sum_splits", "dx_sum_splits")

    def __enter__(self):
        _check(_lib.qlora_timing_reset(), "qlora_timing_reset")
        _check(_lib.qlora_timing_enable(1), "qlora_timing_enable")
        return self

    def __exit__(self, *exc):
        _lib.qlora_timing_enable(0)
        _check(_lib.qlora_timing_collect(), "qlora_timing_collect")
        return False

    @staticmethod
    def totals() -> dict:
        out = {}
        for n in kernel_timing.NAMES:
            ms, cnt = ctypes.c_double(), _i64()
            _check(_lib.qlora_timing_query(n.encode(), ctypes.byref(ms), ctypes.byref(cnt)),
                   "qlora_timing_query")
            if cnt.value:
                out[n] = (ms.value, cnt.value)
        return out


__all__ = ["kernel_timing", "NF4Weight", "QloraError", "quantize", "forward", "backward", "merge", "unmerge",
           "quantize_sections", "forward_sections", "backward_sections", "forward_multi", "forward_dropout",
           "backward_dropout", "backward_noalloc", "adam_step", "nf4_levels", "nf4_sizes", "lib", "EXPORTED", "LIB_PATH"]
