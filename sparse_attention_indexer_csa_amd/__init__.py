"""MI355X (gfx950) CSA indexer score and top-k selection.

Thin ctypes binding over ``libcsa_index.so`` (the C ABI in
``include/csa_index.h``).  Every step of the computation runs in the HIP
kernels; this module only turns torch tensors into pointers, strides and the
current HIP stream, and status codes into exceptions.  PyTorch is used for
device memory and streams only.

Entry points (same names as the C ABI):

* :func:`score`  -> masked scores ``[B,S,W]`` fp32 (-inf where masked)
* :func:`topk`   -> top-k indices of a score matrix
* :func:`select` -> fused score + top-k, ``[B,S,top_k]`` int32 (optionally the scores)
* :func:`score_backward` -> ``(dq, dk, dw)`` fp32, the gradients of
  ``sum(grad * score)`` over unmasked pairs
* :func:`workspace_size`, :func:`backward_workspace_size`, :func:`resolve_plan`

Tensor layouts: ``q [B,H,S,D]`` (any strides with D contiguous, e.g. a
permuted view of a sequence-major ``[B,S,H,D]`` tensor), ``k [B,W,D]``,
``w [B,S,H]``, all ``torch.bfloat16`` on the GPU.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa_index.so")

PLANS = {"auto": 0, "row_tiles": 1, "split_rows": 2}

_OK, _INVALID, _UNSUPPORTED, _WORKSPACE, _DEVICE = range(5)


class CsaIndexError(RuntimeError):
    """A device / launch error reported by the library."""


class CsaUnsupportedError(ValueError):
    """The kernels do not implement this shape or layout (no fallback exists)."""


class _Problem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("S", ctypes.c_int32), ("H", ctypes.c_int32), ("D", ctypes.c_int32),
        ("W", ctypes.c_int32), ("compress_rate", ctypes.c_int32), ("scale", ctypes.c_float),
        ("plan", ctypes.c_int32),
        ("q_sb", ctypes.c_int64), ("q_sh", ctypes.c_int64), ("q_ss", ctypes.c_int64),
        ("k_sb", ctypes.c_int64), ("k_sw", ctypes.c_int64),
        ("w_sb", ctypes.c_int64), ("w_ss", ctypes.c_int64),
    ]


class _Masks(ctypes.Structure):
    _fields_ = [("q_offset", ctypes.c_void_p), ("q_seg", ctypes.c_void_p), ("k_seg", ctypes.c_void_p)]


# Every symbol the header declares, with its ctypes signature.
_VP, _I32, _I64, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
SIGNATURES = {
    "csa_index_score": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    "csa_index_topk": (_I32, [_I64, _I32, _I32, _VP, _VP, _VP, _SZ, _VP]),
    "csa_index_topk_workspace_size": (_I32, [_I64, _I32, _I32, ctypes.POINTER(_SZ)]),
    "csa_index_select": (_I32, [_VP, _VP, _VP, _VP, _VP, _I32, _VP, _VP, _VP, _SZ, _VP]),
    "csa_index_workspace_size": (_I32, [_VP, _I32, ctypes.POINTER(_SZ)]),
    "csa_index_select_noalloc": (_I32, [_VP, _VP, _VP, _VP, _VP, _I32, _VP, _VP, _VP]),
    "csa_index_kl_loss": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    "csa_index_resolve_plan": (_I32, [_VP]),
    "csa_index_score_backward": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "csa_index_backward_workspace_size": (_I32, [_VP, ctypes.POINTER(_SZ)]),
    "csa_status_string": (ctypes.c_char_p, [_I32]),
    "csa_last_error": (ctypes.c_char_p, []),
    "csa_index_abi_version": (_I32, []),
}

ABI_VERSION = 1

_lib = None


def load_library(path: str = LIB_PATH):
    """Load the HIP library; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m sparse_attention_indexer_csa_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.csa_index_abi_version() != ABI_VERSION:
        raise ImportError("libcsa_index.so ABI version mismatch; rebuild it")
    _lib = lib
    return lib


def _raise(status: int, what: str):
    lib = load_library()
    detail = lib.csa_last_error().decode()
    msg = f"{what}: {lib.csa_status_string(status).decode()}: {detail}"
    if status == _UNSUPPORTED:
        raise CsaUnsupportedError(msg)
    if status in (_INVALID, _WORKSPACE):
        raise ValueError(msg)
    raise CsaIndexError(msg)


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dev_tensor(t, name, dtype, ndim):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (the library has no CPU path)")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {tuple(t.shape)}")
    return t


def _strides(t: torch.Tensor):
    """Element strides as the kernels read them: a dimension of size 1 is never
    stepped over (stride 0), and an empty tensor is described as dense."""
    if t.numel() == 0:
        st, acc = [], 1
        for n in reversed(t.shape):
            st.append(acc)
            acc *= max(int(n), 1)
        return tuple(reversed(st))
    return tuple(0 if n == 1 else s for n, s in zip(t.shape, t.stride()))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _problem(q, k, w, compress_rate, scale, plan):
    _dev_tensor(q, "q", torch.bfloat16, 4)
    _dev_tensor(k, "k", torch.bfloat16, 3)
    _dev_tensor(w, "w", torch.bfloat16, 3)
    B, H, S, D = q.shape
    W = k.shape[1]
    if k.shape[0] != B or k.shape[2] != D:
        raise ValueError(f"k must be [B={B}, W, D={D}], got {tuple(k.shape)}")
    if tuple(w.shape) != (B, S, H):
        raise ValueError(f"w must be [B,S,H]=({B},{S},{H}), got {tuple(w.shape)}")
    qs, ks, ws = _strides(q), _strides(k), _strides(w)
    if (D > 1 and qs[3] != 1) or (D > 1 and ks[2] != 1) or (H > 1 and ws[2] != 1):
        raise ValueError("the innermost dimension of q, k (D) and w (H) must be contiguous")
    if not (q.device == k.device == w.device):
        raise ValueError("q, k and w must be on the same device")
    if plan not in PLANS:
        raise ValueError(f"plan must be one of {sorted(PLANS)}")
    p = _Problem(B, S, H, D, W, int(compress_rate), float(scale), PLANS[plan],
                 qs[0], qs[1], qs[2], ks[0], ks[1], ws[0], ws[1])
    return p


def check_mask_shapes(B: int, S: int, W: int, q_offset=None, q_seg=None, k_seg=None) -> None:
    """Shape, dtype and layout checks of the optional mask tensors (no device
    access): q_offset [B], q_seg [B,S], k_seg [B,W], all contiguous int32, and
    q_seg and k_seg both given or both omitted.  The kernels read every one of
    these elements, so a short tensor is refused here, before any launch."""
    for name, t, shape in (("q_offset", q_offset, (B,)), ("q_seg", q_seg, (B, S)), ("k_seg", k_seg, (B, W))):
        if t is None:
            continue
        if not isinstance(t, torch.Tensor) or t.dtype != torch.int32:
            raise ValueError(f"{name} must be an int32 tensor")
        if tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {list(shape)} int32 tensor, got {tuple(t.shape)}")
    if (q_seg is None) != (k_seg is None):
        raise ValueError("q_seg and k_seg must be given together")


def _masks(q, k, q_offset, q_seg, k_seg):
    B, _, S, _ = q.shape
    W = k.shape[1]
    for name, t in (("q_offset", q_offset), ("q_seg", q_seg), ("k_seg", k_seg)):
        if t is not None:
            _dev_tensor(t, name, torch.int32, t.dim())
            if t.device != q.device:
                raise ValueError(f"{name} must be on the device of q")
    check_mask_shapes(B, S, W, q_offset, q_seg, k_seg)
    return _Masks(q_offset.data_ptr() if q_offset is not None else None,
                  q_seg.data_ptr() if q_seg is not None else None,
                  k_seg.data_ptr() if k_seg is not None else None)


def resolve_plan(q, k, w, compress_rate: int, plan: str = "auto") -> str:
    """Name of the plan the library runs for these tensors."""
    lib = load_library()
    p = _problem(q, k, w, compress_rate, 1.0, plan)
    r = lib.csa_index_resolve_plan(ctypes.byref(p))
    if r < 0:
        _raise(_INVALID, "resolve_plan")
    return {v: n for n, v in PLANS.items()}[r]


def workspace_size(q, k, w, top_k: int, compress_rate: int, plan: str = "auto") -> int:
    lib = load_library()
    p = _problem(q, k, w, compress_rate, 1.0, plan)
    n = ctypes.c_size_t(0)
    st = lib.csa_index_workspace_size(ctypes.byref(p), int(top_k), ctypes.byref(n))
    if st != _OK:
        _raise(st, "csa_index_workspace_size")
    return n.value


def score(q, k, w, compress_rate: int, scale: float = 1.0, q_offset=None, q_seg=None, k_seg=None,
          plan: str = "auto", out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Masked indexer scores [B,S,W] fp32 (csa_index_score)."""
    lib = load_library()
    p = _problem(q, k, w, compress_rate, scale, plan)
    m = _masks(q, k, q_offset, q_seg, k_seg)
    if out is None:
        out = torch.empty((p.B, p.S, p.W), dtype=torch.float32, device=q.device)
    else:
        _dev_tensor(out, "out", torch.float32, 3)
        if tuple(out.shape) != (p.B, p.S, p.W) or not out.is_contiguous():
            raise ValueError("out must be a contiguous [B,S,W] float32 tensor")
    st = lib.csa_index_score(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(w), ctypes.byref(m), _ptr(out),
                             ctypes.c_void_p(_stream(q.device)))
    if st != _OK:
        _raise(st, "csa_index_score")
    return out


def topk(scores: torch.Tensor, top_k: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Top-k indices of each row of ``scores[..., W]`` (csa_index_topk); -inf/NaN never chosen."""
    lib = load_library()
    if not isinstance(scores, torch.Tensor) or not scores.is_cuda or scores.dtype != torch.float32:
        raise ValueError("scores must be a float32 GPU tensor")
    if scores.dim() < 1 or not scores.is_contiguous():
        raise ValueError("scores must be contiguous with entries in the last dimension")
    W = scores.shape[-1]
    rows = math.prod(scores.shape[:-1])
    if out is None:
        out = torch.empty((*scores.shape[:-1], int(top_k)), dtype=torch.int32, device=scores.device)
    elif out.dtype != torch.int32 or not out.is_contiguous() or tuple(out.shape) != (*scores.shape[:-1], int(top_k)):
        raise ValueError("out must be a contiguous int32 [..., top_k] tensor")
    st = lib.csa_index_topk(rows, W, int(top_k), _ptr(scores), _ptr(out), None, 0,
                            ctypes.c_void_p(_stream(scores.device)))
    if st != _OK:
        _raise(st, "csa_index_topk")
    return out


def select(q, k, w, top_k: int, compress_rate: int, scale: float = 1.0, q_offset=None, q_seg=None, k_seg=None,
           plan: str = "auto", return_scores: bool = False, out: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None):
    """Fused score + top-k (csa_index_select): idx [B,S,top_k] int32, and scores if asked."""
    lib = load_library()
    p = _problem(q, k, w, compress_rate, scale, plan)
    m = _masks(q, k, q_offset, q_seg, k_seg)
    dev = q.device
    if out is None:
        out = torch.empty((p.B, p.S, int(top_k)), dtype=torch.int32, device=dev)
    elif out.dtype != torch.int32 or not out.is_contiguous() or tuple(out.shape) != (p.B, p.S, int(top_k)):
        raise ValueError("out must be a contiguous int32 [B,S,top_k] tensor")
    sc = torch.empty((p.B, p.S, p.W), dtype=torch.float32, device=dev) if return_scores else None
    ws = None
    if workspace is not None:
        # the caller's buffer as is: the library checks its size (no host query per call)
        if not workspace.is_cuda:
            raise ValueError("workspace must be a device tensor")
        ws = workspace
    elif sc is None:
        need = ctypes.c_size_t(0)
        st = lib.csa_index_workspace_size(ctypes.byref(p), int(top_k), ctypes.byref(need))
        if st != _OK:
            _raise(st, "csa_index_workspace_size")
        if need.value > 0:
            ws = torch.empty(need.value, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = lib.csa_index_select(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(w), ctypes.byref(m), int(top_k), _ptr(out),
                              _ptr(sc), _ptr(ws), ws_bytes, ctypes.c_void_p(_stream(dev)))
    if st != _OK:
        _raise(st, "csa_index_select")
    return (out, sc) if return_scores else out


# Bytes of the library's own scratch buffer used by select_noalloc.
NOALLOC_SCRATCH_BYTES = 16 << 20


def select_noalloc(q, k, w, top_k: int, compress_rate: int, out: torch.Tensor, scale: float = 1.0, q_offset=None,
                   q_seg=None, k_seg=None, plan: str = "auto", scores: Optional[torch.Tensor] = None) -> torch.Tensor:
    """csa_index_select_noalloc: the fused select writing into the caller's
    ``out`` [B,S,top_k] int32 (and ``scores`` [B,S,W] fp32 if given), with
    any workspace taken from the library's fixed per-GPU scratch buffer.
    Nothing is allocated here or in the library.  Calls that overlap on one
    GPU race on that buffer."""
    lib = load_library()
    p = _problem(q, k, w, compress_rate, scale, plan)
    m = _masks(q, k, q_offset, q_seg, k_seg)
    _dev_tensor(out, "out", torch.int32, 3)
    if tuple(out.shape) != (p.B, p.S, int(top_k)) or not out.is_contiguous():
        raise ValueError("out must be a contiguous int32 [B,S,top_k] tensor")
    if scores is not None:
        _dev_tensor(scores, "scores", torch.float32, 3)
        if tuple(scores.shape) != (p.B, p.S, p.W) or not scores.is_contiguous():
            raise ValueError("scores must be a contiguous float32 [B,S,W] tensor")
    st = lib.csa_index_select_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(w), ctypes.byref(m), int(top_k),
                                      _ptr(out), _ptr(scores), ctypes.c_void_p(_stream(q.device)))
    if st != _OK:
        _raise(st, "csa_index_select_noalloc")
    return out


def kl_loss(q, k, w, target, compress_rate: int, scale: float = 1.0, q_offset=None, q_seg=None, k_seg=None,
            grad: bool = False, out: Optional[torch.Tensor] = None, grad_out: Optional[torch.Tensor] = None):
    """Indexer loss (csa_index_kl_loss): per row, KL(target || softmax(score))
    over the visible entries, the target L1-normalised there.  target is
    [B,S,W] fp32.  Returns kl [B,S] fp32, and with grad=True also
    d kl / d score [B,S,W] fp32 (input to score_backward)."""
    lib = load_library()
    p = _problem(q, k, w, compress_rate, scale, "auto")
    m = _masks(q, k, q_offset, q_seg, k_seg)
    dev = q.device
    _dev_tensor(target, "target", torch.float32, 3)
    if tuple(target.shape) != (p.B, p.S, p.W) or not target.is_contiguous():
        raise ValueError("target must be a contiguous [B,S,W] float32 tensor")
    if out is None:
        out = torch.empty((p.B, p.S), dtype=torch.float32, device=dev)
    elif out.dtype != torch.float32 or tuple(out.shape) != (p.B, p.S) or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 [B,S] tensor")
    g = None
    if grad:
        g = grad_out if grad_out is not None else torch.empty((p.B, p.S, p.W), dtype=torch.float32, device=dev)
        _dev_tensor(g, "grad_out", torch.float32, 3)
        if tuple(g.shape) != (p.B, p.S, p.W) or not g.is_contiguous():
            raise ValueError("grad_out must be a contiguous float32 [B,S,W] tensor")
    st = lib.csa_index_kl_loss(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(w), ctypes.byref(m), _ptr(target),
                               _ptr(out), _ptr(g), ctypes.c_void_p(_stream(dev)))
    if st != _OK:
        _raise(st, "csa_index_kl_loss")
    return (out, g) if grad else out


def backward_workspace_size(q, k, w, compress_rate: int) -> int:
    """Bytes of workspace csa_index_score_backward needs for these tensors."""
    lib = load_library()
    p = _problem(q, k, w, compress_rate, 1.0, "auto")
    n = ctypes.c_size_t(0)
    st = lib.csa_index_backward_workspace_size(ctypes.byref(p), ctypes.byref(n))
    if st != _OK:
        _raise(st, "csa_index_backward_workspace_size")
    return n.value


def score_backward(q, k, w, grad, compress_rate: int, scale: float = 1.0, q_offset=None, q_seg=None, k_seg=None,
                   workspace: Optional[torch.Tensor] = None, dq: Optional[torch.Tensor] = None,
                   dk: Optional[torch.Tensor] = None, dw: Optional[torch.Tensor] = None):
    """Gradients (dq [B,H,S,D], dk [B,W,D], dw [B,S,H], fp32) of sum(grad * score)
    over unmasked pairs (csa_index_score_backward); grad is [B,S,W] fp32."""
    lib = load_library()
    p = _problem(q, k, w, compress_rate, scale, "auto")
    m = _masks(q, k, q_offset, q_seg, k_seg)
    dev = q.device
    _dev_tensor(grad, "grad", torch.float32, 3)
    if tuple(grad.shape) != (p.B, p.S, p.W) or not grad.is_contiguous():
        raise ValueError("grad must be a contiguous [B,S,W] float32 tensor")

    def out(t, name, shape):
        if t is None:
            return torch.empty(shape, dtype=torch.float32, device=dev)
        _dev_tensor(t, name, torch.float32, len(shape))
        if tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 tensor of shape {shape}")
        return t

    dq = out(dq, "dq", (p.B, p.H, p.S, p.D))
    dk = out(dk, "dk", (p.B, p.W, p.D))
    dw = out(dw, "dw", (p.B, p.S, p.H))
    ws = None
    if workspace is not None:
        # the caller's buffer as is: the library checks its size (no host query per call)
        if not workspace.is_cuda:
            raise ValueError("workspace must be a device tensor")
        ws = workspace
    else:
        need = ctypes.c_size_t(0)
        st = lib.csa_index_backward_workspace_size(ctypes.byref(p), ctypes.byref(need))
        if st != _OK:
            _raise(st, "csa_index_backward_workspace_size")
        if need.value > 0:
            ws = torch.empty(need.value, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = lib.csa_index_score_backward(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(w), ctypes.byref(m), _ptr(grad),
                                      _ptr(dq), _ptr(dk), _ptr(dw), _ptr(ws), ws_bytes,
                                      ctypes.c_void_p(_stream(dev)))
    if st != _OK:
        _raise(st, "csa_index_score_backward")
    return dq, dk, dw


__all__ = ["score", "topk", "select", "select_noalloc", "kl_loss", "score_backward", "workspace_size", "backward_workspace_size",
           "resolve_plan", "load_library", "CsaIndexError",
           "CsaUnsupportedError", "LIB_PATH", "SIGNATURES", "PLANS"]
