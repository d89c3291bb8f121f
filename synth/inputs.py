"""Seeded, synthetic indexer workloads.

Layouts follow the head-major indexer tensors of the fused StreamIndex kernel
(MaxText PR #5079 "Add StreamIndex Kernel for CSA", inline review on the
BlockSpecs): queries ``q[B,H,S,D]``, compressed keys ``k[B,W,D]`` shared by all
heads, head weights ``w[B,S,H]``.  Values are bfloat16, stored here as their
16-bit patterns (``numpy.uint16``) so that the CPU oracle and the GPU library
consume the very same bits.

Draw order for one seed (numpy ``default_rng`` = PCG64, C order): q, then k,
then w, then segment structure / decode lengths.  Large tensors are drawn in
batch slices; numpy's generators produce the same stream whether a tensor is
drawn at once or slice by slice, so the slicing only bounds host memory.

Distributions:

* ``"gauss"``: q, k ~ N(0,1)/sqrt(D); w ~ N(0,1)/sqrt(H); drawn in float32,
  rounded to bfloat16 (round to nearest, ties to even).
* ``"int"``: the integer grid.  q, k are integers uniform in [-4, 4] times
  2^-3; w is integers uniform in [-8, 8] times 2^-4.  Every such value is exact
  in bfloat16 and every partial sum of the score is exact in float32 for the
  shapes used here (D <= 128, H <= 64).

Segments (packed documents): each batch row packs ``n_docs ~ U{1..6}``
documents; the ``n_docs - 1`` cut points are distinct values drawn uniformly
from ``{1..S-1}`` (or from the multiples of the compress rate for the aligned
variant) and sorted.  ``q_seg[b,i]`` is the index of the document holding token
``i``.  Compressed entry ``j`` covers tokens ``j*m .. j*m+m-1`` and takes the
segment of its last token, ``k_seg[b,j] = q_seg[b, min((j+1)*m-1, S-1)]``.

Decode: one query row per sequence, valid compressed length
``L_b ~ U{lo..hi}``; the row's absolute position is ``q_offset[b] = m*L_b - 1``.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input values are outside the generator's contract")
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Problem:
    """One indexer workload.  Arrays are host numpy arrays, dense, C order."""

    name: str
    B: int
    S: int
    H: int
    D: int
    W: int
    m: int  # compress rate
    top_k: int
    scale: float
    q: np.ndarray  # uint16 [B,H,S,D] bf16 bits
    k: np.ndarray  # uint16 [B,W,D]
    w: np.ndarray  # uint16 [B,S,H]
    q_offset: Optional[np.ndarray] = None  # int32 [B]
    q_seg: Optional[np.ndarray] = None  # int32 [B,S]
    k_seg: Optional[np.ndarray] = None  # int32 [B,W]
    seed: Optional[int] = None
    meta: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        return self.B * self.S


def _draw_bf16(rng, shape, dist, sigma, grid_lo, grid_hi, grid_scale, slice_axis0=True):
    out = np.empty(shape, dtype=np.uint16)
    n0 = shape[0] if slice_axis0 else 1
    for b in range(n0):
        sub = shape[1:] if slice_axis0 else shape
        if dist == "gauss":
            v = rng.standard_normal(sub, dtype=np.float32) * np.float32(sigma)
        elif dist == "int":
            v = rng.integers(grid_lo, grid_hi + 1, size=sub, dtype=np.int8).astype(np.float32) * np.float32(grid_scale)
        elif dist == "zeros":
            v = np.zeros(sub, dtype=np.float32)
        else:
            raise ValueError(f"unknown distribution {dist!r}")
        if slice_axis0:
            out[b] = f32_to_bf16_bits(v)
        else:
            out[...] = f32_to_bf16_bits(v)
    return out


def _segments(rng, B, S, m, aligned, max_docs=6):
    q_seg = np.zeros((B, S), dtype=np.int32)
    for b in range(B):
        n_docs = int(rng.integers(1, max_docs + 1))
        if aligned:
            pool = np.arange(1, S // m, dtype=np.int64) * m
        else:
            pool = np.arange(1, S, dtype=np.int64)
        n_cuts = min(n_docs - 1, len(pool))
        cuts = np.sort(rng.choice(pool, size=n_cuts, replace=False)) if n_cuts > 0 else np.zeros(0, np.int64)
        q_seg[b] = np.searchsorted(cuts, np.arange(S), side="right").astype(np.int32)
    return q_seg


def _entry_segments(q_seg, W, m):
    B, S = q_seg.shape
    last_tok = np.minimum((np.arange(W, dtype=np.int64) + 1) * m - 1, S - 1)
    return np.ascontiguousarray(q_seg[:, last_tok]).astype(np.int32)


def make_problem(
    B: int,
    S: int,
    H: int,
    D: int,
    W: int,
    m: int,
    top_k: int,
    *,
    dist: str = "gauss",
    seed: int = 0,
    scale: float = 1.0,
    segments: Optional[str] = None,  # None | "random" | "aligned"
    decode_lengths: Optional[tuple] = None,  # (lo, hi): S must be 1
    q_offset: Optional[np.ndarray] = None,
    name: str = "custom",
) -> Problem:
    """Draw one seeded workload.  See the module docstring for the recipe."""
    rng = np.random.default_rng(seed)
    q = _draw_bf16(rng, (B, H, S, D), dist, 1.0 / math.sqrt(D), -4, 4, 2.0 ** -3)
    k = _draw_bf16(rng, (B, W, D), dist, 1.0 / math.sqrt(D), -4, 4, 2.0 ** -3)
    w = _draw_bf16(rng, (B, S, H), dist, 1.0 / math.sqrt(H), -8, 8, 2.0 ** -4)
    q_seg = k_seg = None
    meta = {}
    if segments is not None:
        if segments not in ("random", "aligned"):
            raise ValueError(segments)
        q_seg = _segments(rng, B, S, m, aligned=(segments == "aligned"))
        k_seg = _entry_segments(q_seg, W, m)
        meta["segments"] = segments
    if decode_lengths is not None:
        if S != 1:
            raise ValueError("decode workloads have one query row per sequence")
        lo, hi = decode_lengths
        L = rng.integers(lo, hi + 1, size=B).astype(np.int64)
        q_offset = (m * L - 1).astype(np.int32)
        meta["valid_len"] = L.astype(np.int64)
    elif q_offset is not None:
        q_offset = np.asarray(q_offset, dtype=np.int32).reshape(B)
    return Problem(
        name=name, B=B, S=S, H=H, D=D, W=W, m=m, top_k=top_k, scale=float(scale),
        q=q, k=k, w=w, q_offset=q_offset, q_seg=q_seg, k_seg=k_seg, seed=seed, meta=meta,
    )


# The indexer workloads.  Shapes follow the seq-16384 DeepSeek-V4 indexer
# (64 heads of width 128, compress rate 4, top-512 selection); the small ones
# exist for exact parity, the decode one for the cache-streaming path.
CONFIGS = {
    "c1": dict(B=1, S=256, H=4, D=32, W=64, m=4, top_k=16, dist="int", seed=1),
    "c2": dict(B=1, S=4096, H=64, D=128, W=1024, m=4, top_k=512, dist="gauss", seed=2),
    "c2int": dict(B=1, S=4096, H=64, D=128, W=1024, m=4, top_k=512, dist="int", seed=22),
    "c3": dict(B=1, S=16384, H=64, D=128, W=4096, m=4, top_k=512, dist="gauss", seed=3),
    "c4": dict(B=4, S=8192, H=64, D=128, W=2048, m=4, top_k=512, dist="gauss", seed=4, segments="random"),
    "c4aligned": dict(B=4, S=8192, H=64, D=128, W=2048, m=4, top_k=512, dist="gauss", seed=4, segments="aligned"),
    "c5": dict(B=64, S=1, H=64, D=128, W=32768, m=4, top_k=512, dist="gauss", seed=5,
               decode_lengths=(4096, 32768)),
}

CONFIG_TITLES = {
    "c1": "tiny prefill, integer grid (B=1 S=256 H=4 D=32 m=4 W=64 k=16)",
    "c2": "mid prefill (B=1 S=4096 H=64 D=128 m=4 W=1024 k=512)",
    "c2int": "mid prefill, integer grid (B=1 S=4096 H=64 D=128 m=4 W=1024 k=512)",
    "c3": "long prefill seq 16384 (B=1 S=16384 H=64 D=128 m=4 W=4096 k=512)",
    "c4": "packed-segment prefill (B=4 S=8192 H=64 D=128 m=4 W=2048 k=512, 1-6 docs/row)",
    "c4aligned": "packed-segment prefill, m-aligned documents",
    "c5": "decode (B=64 S=1 H=64 D=128 W_cache=32768, L_b~U[4096,32768], k=512)",
}


def make_config(name: str, seed: Optional[int] = None) -> Problem:
    """Build one of the named workloads (optionally with another seed)."""
    cfg = dict(CONFIGS[name])
    if seed is not None:
        cfg["seed"] = seed
    return make_problem(name=name, **cfg)
