"""Seeded synthetic workloads for the Veda hot path.

This module holds *inputs only*: sequence geometry (spans and grids), budget
requests, and seeded random tensors. It holds none of the method's
arithmetic (no tile shapes are chosen here, no budgets are split, nothing is
pooled, scored or selected). Both the CPU oracle and the HIP path take their
inputs from here.

The five workloads mirror the shapes the Veda pages quote: a 104k-token
layer comparable to 1344x768 at 124 frames (the headline), a 720p 241-frame
clip with per-head tile shapes, and three smaller cases. The pages measure on
real MiniMax H3 / Waver activations, which are not available; these synthetic
tensors stand in for them, by the recipe below.

Recipe (per workload, seed ``1000 + index``, numpy PCG64):
  1. q, k, v: float32 standard normal, shape [S, H, D]. Rows are drawn in
     chunks of 4096; chunk c of tensor i (q=0, k=1, v=2) comes from its own
     generator seeded with SeedSequence(seed, spawn_key=(i, c)), so chunks can
     be drawn in parallel and the values do not depend on the thread count.
     Everything below comes from one generator seeded with `seed`.
  2. positional-bias parameters (workloads with ``bias=True``): 4 frequency
     triples drawn uniformly from {0,1,2}^3 minus the zero triple, 4 phases
     U[0, 2*pi), and per-head mixing C ~ N(0, 1/4) of shape [H, 8, D].
     B(t,h,w) = [cos th_m, sin th_m]_{m=1..4} @ C_h with
     th_m = 2*pi*(ft*t/T + fh*h/Hg + fw*w/Wg) + phi_m over each video span's
     own grid; q and k of video rows get + 0.5 * B (the same B for both).
  3. predictor projections [H, 3D, D]:
       'gauss'  : N(0, 1/(3D)), rounded to bf16 values;
       'embed16': W_q, W_k ~ N(0, 1/D) of shape [H, D, 16]; P_q holds
                  W_q W_k^T - I in its first D rows and zeros below, P_k = 0.
                  With the residual mean this gives score ~ (m_q W_q).(m_k W_k).
  4. bf16 workloads: q, k, v are rounded to bf16 (round to nearest even);
     the same bf16 values go to both sides.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
import math
import os

import numpy as np

__all__ = ["Workload", "WORKLOADS", "get", "generate", "Inputs", "bf16_round",
           "bf16_bits", "sample_tiles"]


@dataclass(frozen=True)
class Workload:
    """Geometry and budget request of one synthetic attention layer.

    ``refs``       : ((start, (T, H, W)), ...) reference video spans, packed order.
    ``target``     : (start, (T, H, W)) the generated video span (packed last).
    ``head_shapes``: per head, the target's tile box (t, h, w), or None to ask
                     for the least-padding box.
    ``generated`` / ``reference``: budget requests ('sparsity', s) |
                     ('ratio', r) | ('tiles', n).
    Rows outside every span (text / condition tokens) are global rows.
    """
    name: str
    index: int
    seq_len: int
    n_heads: int
    head_dim: int
    dtype: str                      # 'f32' or 'bf16'
    refs: tuple
    target: tuple
    head_shapes: tuple
    generated: tuple
    reference: tuple
    bias: bool
    proj: str                       # 'gauss' or 'embed16'
    note: str = ""

    @property
    def seed(self) -> int:
        return 1000 + self.index

    @property
    def n_video_rows(self) -> int:
        rows = sum(g[0] * g[1] * g[2] for _, g in self.refs)
        g = self.target[1]
        return rows + g[0] * g[1] * g[2]


def _grid_rows(g):
    return g[0] * g[1] * g[2]


WORKLOADS = {
    "tiny": Workload(
        name="tiny", index=1, seq_len=1024, n_heads=2, head_dim=64, dtype="f32",
        refs=(), target=(0, (4, 16, 16)), head_shapes=((2, 8, 8),) * 2,
        generated=("tiles", 2.0), reference=("tiles", 2.0),
        bias=False, proj="embed16",
        note="8 tiles of (2,8,8); exactly 2 key tiles per query tile"),
    "padding": Workload(
        name="padding", index=2, seq_len=1264, n_heads=4, head_dim=64, dtype="bf16",
        refs=(), target=(0, (5, 12, 20)), head_shapes=(None,) * 4,
        generated=("ratio", 0.25), reference=("ratio", 0.25),
        bias=False, proj="gauss",
        note="1200 video rows in padded tiles plus 64 global text rows"),
    "mid": Workload(
        name="mid", index=3, seq_len=28672, n_heads=24, head_dim=128, dtype="bf16",
        refs=(), target=(0, (16, 32, 56)), head_shapes=(None,) * 24,
        generated=("sparsity", 0.9), reference=("sparsity", 0.9),
        bias=True, proj="gauss",
        note="224 tiles, 90% sparse, positional-locality bias"),
    "headline": Workload(
        name="headline", index=4, seq_len=108448, n_heads=24, head_dim=128, dtype="bf16",
        refs=((0, (1, 48, 84)),), target=(4032, (31, 48, 70)), head_shapes=(None,) * 24,
        generated=("sparsity", 0.9), reference=("sparsity", 0.9),
        bias=True, proj="gauss",
        note="104,160 video rows (1344x768, 124 frames) + 4,032 reference rows "
             "+ 256 global text rows, 90% sparse"),
    "headline_iid": Workload(
        name="headline_iid", index=4, seq_len=108448, n_heads=24, head_dim=128, dtype="bf16",
        refs=((0, (1, 48, 84)),), target=(4032, (31, 48, 70)), head_shapes=(None,) * 24,
        generated=("sparsity", 0.9), reference=("sparsity", 0.9),
        bias=False, proj="gauss",
        note="headline geometry with pure N(0,1) q/k (no locality)"),
    "long": Workload(
        name="long", index=5, seq_len=219600, n_heads=24, head_dim=128, dtype="bf16",
        refs=(), target=(0, (61, 45, 80)),
        head_shapes=((1, 8, 16),) * 12 + ((8, 4, 4),) * 12,
        generated=("sparsity", 0.95), reference=("sparsity", 0.95),
        bias=True, proj="gauss",
        note="720p x 241 frames, 95% sparse, spatial and temporal head shapes"),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> float32 holding the nearest bf16 value (ties to even)."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    out = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return out.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 holding bf16 values -> their uint16 bit patterns."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (bits >> np.uint32(16)).astype(np.uint16)


@dataclass
class Inputs:
    """One layer's tensors. Arrays are float32 holding the exact values both
    sides use (bf16-representable for bf16 workloads)."""
    workload: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    proj_q: np.ndarray              # [H, 3D, D] float32
    proj_k: np.ndarray
    extras: dict = field(default_factory=dict)


def _positional_bias(rng, wl: Workload):
    """Low-rank smooth bias over the video spans: [S, H, D] contributions,
    returned as (rows, B) per span to keep memory bounded."""
    triples = [(a, b, c) for a in range(3) for b in range(3) for c in range(3)
               if (a, b, c) != (0, 0, 0)]
    pick = rng.integers(0, len(triples), size=4)
    freqs = np.array([triples[i] for i in pick], dtype=np.float64)   # [4, 3]
    phases = rng.uniform(0.0, 2.0 * math.pi, size=4)
    mix = rng.normal(0.0, 0.5, size=(wl.n_heads, 8, wl.head_dim))   # std 1/2 -> var 1/4
    out = []
    for start, grid in list(wl.refs) + [wl.target]:
        T, Hg, Wg = grid
        t = np.arange(T, dtype=np.float64)[:, None, None] / T
        h = np.arange(Hg, dtype=np.float64)[None, :, None] / Hg
        w = np.arange(Wg, dtype=np.float64)[None, None, :] / Wg
        feats = []
        for m in range(4):
            th = 2.0 * math.pi * (freqs[m, 0] * t + freqs[m, 1] * h + freqs[m, 2] * w) + phases[m]
            feats.append(np.cos(th).reshape(-1))
        for m in range(4):
            th = 2.0 * math.pi * (freqs[m, 0] * t + freqs[m, 1] * h + freqs[m, 2] * w) + phases[m]
            feats.append(np.sin(th).reshape(-1))
        F = np.stack(feats, axis=1).astype(np.float32)                 # [rows, 8]
        M = np.ascontiguousarray(mix.astype(np.float32).transpose(1, 0, 2))
        B = (F @ M.reshape(8, -1)).reshape(F.shape[0], wl.n_heads, wl.head_dim)
        out.append((start, B))
    return out, dict(freqs=freqs, phases=phases)


_CHUNK_ROWS = 4096


def _normal_chunked(seed, tensor, shape):
    """float32 N(0,1) of `shape`, filled in row chunks from per-chunk seeds."""
    out = np.empty(shape, dtype=np.float32)
    n_chunks = -(-shape[0] // _CHUNK_ROWS)

    def fill(c):
        g = np.random.Generator(np.random.PCG64(
            np.random.SeedSequence(seed, spawn_key=(tensor, c))))
        a, b = c * _CHUNK_ROWS, min(shape[0], (c + 1) * _CHUNK_ROWS)
        g.standard_normal(out=out[a:b], dtype=np.float32)

    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    if n_chunks == 1 or workers == 1:
        for c in range(n_chunks):
            fill(c)
    else:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out


def generate(wl: Workload | str) -> Inputs:
    """Draw the workload's tensors from its seed (see the module recipe)."""
    if isinstance(wl, str):
        wl = get(wl)
    rng = np.random.default_rng(wl.seed)
    shape = (wl.seq_len, wl.n_heads, wl.head_dim)
    q, k, v = (_normal_chunked(wl.seed, i, shape) for i in range(3))
    extras = {}
    if wl.bias:
        spans, extras = _positional_bias(rng, wl)
        for start, B in spans:
            n = B.shape[0]
            B *= np.float32(0.5)
            q[start:start + n] += B
            k[start:start + n] += B
            del B
    D = wl.head_dim
    if wl.proj == "gauss":
        pq = rng.normal(0.0, 1.0 / math.sqrt(3 * D), size=(wl.n_heads, 3 * D, D))
        pk = rng.normal(0.0, 1.0 / math.sqrt(3 * D), size=(wl.n_heads, 3 * D, D))
        pq = bf16_round(pq.astype(np.float32))
        pk = bf16_round(pk.astype(np.float32))
    elif wl.proj == "embed16":
        wq = rng.normal(0.0, 1.0 / math.sqrt(D), size=(wl.n_heads, D, 16))
        wk = rng.normal(0.0, 1.0 / math.sqrt(D), size=(wl.n_heads, D, 16))
        pq = np.zeros((wl.n_heads, 3 * D, D), dtype=np.float64)
        pq[:, :D, :] = np.einsum("hde,hfe->hdf", wq, wk) - np.eye(D)[None]
        pq = pq.astype(np.float32)
        pk = np.zeros((wl.n_heads, 3 * D, D), dtype=np.float32)
        extras["w_q"] = wq
        extras["w_k"] = wk
    else:
        raise ValueError(wl.proj)
    if wl.dtype == "bf16":
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    return Inputs(wl, q, k, v, pq, pk, extras)


def sample_tiles(n_tiles: int, count: int, seed: int) -> np.ndarray:
    """A seeded, sorted sample of query-tile indices for sampled parity checks."""
    rng = np.random.default_rng(seed)
    count = min(count, n_tiles)
    return np.sort(rng.choice(n_tiles, size=count, replace=False))
