"""Python face of the CPU oracle (``csa_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the library.  It shares no code with the
HIP path.  ``build()`` compiles the C file with gcc (OpenMP, ``-ffp-contract=off``
so that no multiply-add is fused); the shared object lives in ``oracle/_build``.

All functions take a :class:`synth.Problem` (bf16 bit patterns, head-major q)
and return numpy arrays.
"""

from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csa_oracle.c")
_BUILD = os.path.join(_HERE, "_build")
_SO = os.path.join(_BUILD, "libcsa_oracle.so")

# x86-64-v3 (AVX2/FMA) keeps the object runnable on any recent host; the
# contraction switch keeps every multiply and add separately rounded.
CFLAGS = ["-O3", "-march=x86-64-v3", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
          "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra"]

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle; returns the path of the shared object."""
    os.makedirs(_BUILD, exist_ok=True)
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + f".tmp{os.getpid()}"
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_SO)
    i64, f32, f64, vp = ctypes.c_int64, ctypes.c_float, ctypes.c_double, ctypes.c_void_p
    lib.csa_oracle_scores_f32.argtypes = [i64] * 6 + [f32] + [vp] * 6 + [i64, vp, vp]
    lib.csa_oracle_scores_f32.restype = None
    lib.csa_oracle_scores_f64.argtypes = [i64] * 6 + [f64] + [vp] * 6 + [i64, vp, vp]
    lib.csa_oracle_scores_f64.restype = None
    lib.csa_oracle_valid.argtypes = [i64, i64, i64, vp, vp, vp, i64, vp, vp]
    lib.csa_oracle_valid.restype = None
    lib.csa_oracle_topk.argtypes = [i64, i64, i64, vp, vp]
    lib.csa_oracle_topk.restype = None
    lib.csa_oracle_backward_f64.argtypes = [i64] * 6 + [f64] + [vp] * 13
    lib.csa_oracle_backward_f64.restype = None
    lib.csa_oracle_backward_sample_f64.argtypes = [i64] * 6 + [f64] + [vp] * 7 + [i64, vp, i64, vp] + [vp] * 6
    lib.csa_oracle_backward_sample_f64.restype = None
    lib.csa_oracle_kl_from_scores.argtypes = [i64, i64, vp, vp, vp, vp, vp]
    lib.csa_oracle_kl_from_scores.restype = None
    lib.csa_oracle_version.restype = ctypes.c_int
    lib.csa_oracle_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _rows_arg(P, rows):
    if rows is None:
        return P.B * P.S, None
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
    if r.size and (r.min() < 0 or r.max() >= P.B * P.S):
        raise ValueError("row id out of range")
    return int(r.size), r


def _check(P):
    for name, arr, shape in (("q", P.q, (P.B, P.H, P.S, P.D)), ("k", P.k, (P.B, P.W, P.D)),
                             ("w", P.w, (P.B, P.S, P.H))):
        if tuple(arr.shape) != shape or arr.dtype != np.uint16:
            raise ValueError(f"{name}: expected uint16 {shape}, got {arr.dtype} {arr.shape}")
    if (P.q_seg is None) != (P.k_seg is None):
        raise ValueError("q_seg and k_seg go together")
    if P.m < 1:
        raise ValueError("compress rate must be >= 1")


def scores(P, rows: Optional[Sequence[int]] = None, precision: str = "f32") -> np.ndarray:
    """Masked scores of the given rows (b*S+i), shape [n_rows, W]; -inf = masked."""
    _check(P)
    lib = _load()
    n, r = _rows_arg(P, rows)
    q, k, w = _c(P.q, np.uint16), _c(P.k, np.uint16), _c(P.w, np.uint16)
    qo, qs, ks = _c(P.q_offset, np.int32), _c(P.q_seg, np.int32), _c(P.k_seg, np.int32)
    args = (P.B, P.S, P.H, P.D, P.W, P.m)
    if precision == "f32":
        out = np.empty((n, P.W), dtype=np.float32)
        lib.csa_oracle_scores_f32(*args, float(P.scale), _ptr(q), _ptr(k), _ptr(w), _ptr(qo),
                                  _ptr(qs), _ptr(ks), n, _ptr(r), _ptr(out))
    elif precision == "f64":
        out = np.empty((n, P.W), dtype=np.float64)
        lib.csa_oracle_scores_f64(*args, float(P.scale), _ptr(q), _ptr(k), _ptr(w), _ptr(qo),
                                  _ptr(qs), _ptr(ks), n, _ptr(r), _ptr(out))
    else:
        raise ValueError(precision)
    return out


def valid(P, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Boolean candidate mask of the given rows, shape [n_rows, W]."""
    lib = _load()
    n, r = _rows_arg(P, rows)
    out = np.empty((n, P.W), dtype=np.uint8)
    lib.csa_oracle_valid(P.S, P.W, P.m, _ptr(_c(P.q_offset, np.int32)), _ptr(_c(P.q_seg, np.int32)),
                         _ptr(_c(P.k_seg, np.int32)), n, _ptr(r), _ptr(out))
    return out.astype(bool)


def topk(score_rows: np.ndarray, top_k: int) -> np.ndarray:
    """Top-k indices of each row of a [rows, W] float32 matrix (-inf/NaN never chosen)."""
    s = np.ascontiguousarray(score_rows, dtype=np.float32)
    if s.ndim != 2:
        raise ValueError("expected [rows, W]")
    if top_k < 1:
        raise ValueError("top_k must be >= 1")
    out = np.empty((s.shape[0], top_k), dtype=np.int32)
    _load().csa_oracle_topk(s.shape[0], s.shape[1], top_k, _ptr(s), _ptr(out))
    return out


def threads() -> int:
    """Number of OpenMP threads the oracle runs on."""
    return int(_load().csa_oracle_threads())


def select(P, rows: Optional[Sequence[int]] = None):
    """(scores [n_rows, W] fp32, idx [n_rows, top_k] int32) of the given rows."""
    s = scores(P, rows)
    return s, topk(s, P.top_k)


def backward(P, g: np.ndarray, stats: bool = False):
    """Gradients of sum(g * score) over unmasked (i, j), float64.

    g is the upstream gradient of the scores, [B, S, W] float32 (its values at
    masked positions are ignored).  Returns (dq [B,H,S,D], dk [B,W,D],
    dw [B,S,H]); with stats=True also (sq, sk, sw), the same shapes with a
    last axis of 3 per element: the sum of |term| and of term^2 over the
    terms whose ReLU derivative is decided, and the undecided mass (see
    csa_oracle.c).  error_bounds() turns them into bounds.
    """
    _check(P)
    gg = np.ascontiguousarray(g, dtype=np.float32)
    if gg.shape != (P.B, P.S, P.W):
        raise ValueError(f"g: expected {(P.B, P.S, P.W)}, got {gg.shape}")
    lib = _load()
    q, k, w = _c(P.q, np.uint16), _c(P.k, np.uint16), _c(P.w, np.uint16)
    qo, qs, ks = _c(P.q_offset, np.int32), _c(P.q_seg, np.int32), _c(P.k_seg, np.int32)
    dq = np.empty((P.B, P.H, P.S, P.D), np.float64)
    dk = np.empty((P.B, P.W, P.D), np.float64)
    dw = np.empty((P.B, P.S, P.H), np.float64)
    sq = np.empty(dq.shape + (3,)) if stats else None
    sk = np.empty(dk.shape + (3,)) if stats else None
    sw = np.empty(dw.shape + (3,)) if stats else None
    lib.csa_oracle_backward_f64(P.B, P.S, P.H, P.D, P.W, P.m, float(P.scale), _ptr(q), _ptr(k), _ptr(w),
                                _ptr(qo), _ptr(qs), _ptr(ks), _ptr(gg), _ptr(dq), _ptr(dk), _ptr(dw),
                                _ptr(sq), _ptr(sk), _ptr(sw))
    return (dq, dk, dw, sq, sk, sw) if stats else (dq, dk, dw)


def backward_sample(P, g: np.ndarray, rows: Sequence[int], entries: Sequence[int]):
    """The gradients of backward() for chosen rows (b*S+i) and entries (b*W+j):
    (dq [n_rows,H,D], dw [n_rows,H], dk [n_entries,D], sq, sw, sk), float64,
    with the same per-element statistics (last axis 3)."""
    _check(P)
    gg = np.ascontiguousarray(g, dtype=np.float32)
    if gg.shape != (P.B, P.S, P.W):
        raise ValueError(f"g: expected {(P.B, P.S, P.W)}, got {gg.shape}")
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
    e = np.ascontiguousarray(np.asarray(entries, dtype=np.int64).reshape(-1))
    if r.size and (r.min() < 0 or r.max() >= P.B * P.S):
        raise ValueError("row id out of range")
    if e.size and (e.min() < 0 or e.max() >= P.B * P.W):
        raise ValueError("entry id out of range")
    lib = _load()
    q, k, w = _c(P.q, np.uint16), _c(P.k, np.uint16), _c(P.w, np.uint16)
    qo, qs, ks = _c(P.q_offset, np.int32), _c(P.q_seg, np.int32), _c(P.k_seg, np.int32)
    dq = np.empty((r.size, P.H, P.D), np.float64)
    dw = np.empty((r.size, P.H), np.float64)
    dk = np.empty((e.size, P.D), np.float64)
    sq, sw, sk = np.empty(dq.shape + (3,)), np.empty(dw.shape + (3,)), np.empty(dk.shape + (3,))
    lib.csa_oracle_backward_sample_f64(P.B, P.S, P.H, P.D, P.W, P.m, float(P.scale), _ptr(q), _ptr(k), _ptr(w),
                                       _ptr(qo), _ptr(qs), _ptr(ks), _ptr(gg), r.size, _ptr(r), e.size, _ptr(e),
                                       _ptr(dq), _ptr(dw), _ptr(dk), _ptr(sq), _ptr(sw), _ptr(sk))
    return dq, dw, dk, sq, sw, sk


# Unit roundoffs of float32 and bfloat16 (round to nearest).
U_F32 = 2.0 ** -24
U_BF16 = 2.0 ** -9
# Confidence parameter of the bounds (the same value the C oracle uses for
# its logit bound eps_l).
LAMBDA = 8.0


def sum_bound_factor(n: int) -> float:
    """exp(LAMBDA sqrt(n) u + n u^2 / (1 - u)) - 1: a float32 sum of n terms
    lies within this factor times sum|x| of the exact sum with probability at
    least 1 - 2 n exp(-LAMBDA^2 (1 - u)^2 / 2) (Higham and Mary 2019, the
    probabilistic rounding error analysis of summation and inner products)."""
    return math.expm1(LAMBDA * math.sqrt(n) * U_F32 + n * U_F32 * U_F32 / (1.0 - U_F32))


def error_bounds(value: np.ndarray, stats: np.ndarray, n: int, bf16_operand: bool) -> np.ndarray:
    """Per-element bound on |fp32 result - oracle float64 value| of one gradient.

    value: the oracle's float64 gradient; stats: its statistics (last axis:
    sum |t| and sum t^2 over the terms whose ReLU derivative is decided, and
    the undecided mass U); n: the longest chain of float32 additions an
    implementation accumulates for one element; bf16_operand: whether each
    term's gradient operand (g [l>0] for dq, g w [l>0] for dk) is rounded to
    bfloat16 once (round to nearest) before the product.

    bound = U + LAMBDA (u_bf16 + 2u) sqrt(sum t^2) [bf16 operand only]
              + sum_bound_factor(n) sum|t| + 4 u |value|

    The rounding errors of the bf16 operands are independent, bounded by
    u_bf16 (plus u for an fp32 product rounded first) and of mean zero, so
    their weighted sum exceeds LAMBDA (u_bf16 + 2u) sqrt(sum t^2) with
    probability below 2 exp(-LAMBDA^2 / 2) (Hoeffding's inequality).  The
    float32 accumulation is covered by the summation bound, the final
    multiplies (scale, weight) by 4u |value|.  U counts in full every term
    whose fp32 logit may have the other sign (for dw: the most that fp32
    logits can move ReLU(l)).  Each part fails with probability below 1e-9
    per element at the sizes used.
    """
    a, r2, und = stats[..., 0], stats[..., 1], stats[..., 2]
    b = und + sum_bound_factor(n) * a + 4 * U_F32 * np.abs(value)
    if bf16_operand:
        b = b + LAMBDA * (U_BF16 + 2 * U_F32) * np.sqrt(r2)
    return b


def kl_from_scores(score_rows: np.ndarray, target: np.ndarray, grad: bool = False, magnitudes: bool = False):
    """KL(target || softmax(scores)) per row over the visible entries
    (scores -inf where masked), the target normalised over those entries;
    see csa_oracle.c.  score_rows [rows, W] (taken as float64), target
    [rows, W] float32.  Returns kl [rows] float64, then grad [rows, W]
    (d kl / d score) and magnitudes [rows, 3] if asked."""
    s = np.ascontiguousarray(score_rows, dtype=np.float64)
    a = np.ascontiguousarray(target, dtype=np.float32)
    if s.ndim != 2 or a.shape != s.shape:
        raise ValueError("scores and target must both be [rows, W]")
    kl = np.empty(s.shape[0], np.float64)
    g = np.empty(s.shape, np.float64) if grad else None
    mg = np.empty((s.shape[0], 3), np.float64) if magnitudes else None
    _load().csa_oracle_kl_from_scores(s.shape[0], s.shape[1], _ptr(s), _ptr(a), _ptr(kl), _ptr(g), _ptr(mg))
    out = (kl,)
    if grad:
        out += (g,)
    if magnitudes:
        out += (mg,)
    return out if len(out) > 1 else kl


def kl_loss(P, target: np.ndarray, rows: Optional[Sequence[int]] = None, grad: bool = False,
            magnitudes: bool = False):
    """The indexer KL loss of the given rows (b*S+i): the oracle's float32
    scores of those rows, then kl_from_scores with the rows' targets.
    target is [B, S, W]."""
    s = scores(P, rows)
    t = np.asarray(target, dtype=np.float32).reshape(P.B * P.S, P.W)
    if rows is not None:
        t = t[np.asarray(rows, dtype=np.int64).reshape(-1)]
    return kl_from_scores(s, t, grad=grad, magnitudes=magnitudes)
