"""Tile-level teacher map and the recall of a selection (oracle; test
infrastructure only).

The news pages describe Veda's training signal in one sentence: full
attention, max-pooled to tiles, gives a tile-level teacher distribution that
the predictor learns to reproduce (comfyui-wiki Veda news, Spanish edition
§ Qué hace Veda, French edition § Ce que fait Veda). Reading, in the plainest
terms that sentence supports:

  P[i, j]  full attention of head h: softmax over every real key row j of
           q_i . k_j / sqrt(D), for every real query row i;
  T[a, b]  the teacher map: max of P[i, j] over the real rows i of query tile
           a and the real rows j of key tile b (max-pooling the attention map
           onto the packed tiles);
  T^[a, b] the teacher distribution of query tile a: T[a, b] / sum_b T[a, b];
  recall   of a selection (a block mask): for query tile a, the teacher
           distribution's mass on the tiles the mask keeps.

fp64 throughout.
"""
from __future__ import annotations

import numpy as np


def teacher_map(q, k, layout, heads, query_tiles=None):
    """[H', n_q, n_tiles] fp64 max-pooled full attention (T above) for the
    listed query tiles (all when None)."""
    S, _, D = q.shape
    n = layout.n_tiles
    tiles = range(n) if query_tiles is None else list(query_tiles)
    rows_of = [layout.tile_rows(b) for b in range(n)]
    keys = np.concatenate(rows_of)                        # every real row, tile order
    tile_of_key = np.concatenate([np.full(len(r), b) for b, r in enumerate(rows_of)])
    out = np.zeros((len(heads), len(tiles), n), dtype=np.float64)
    for hi, h in enumerate(heads):
        K = k[keys, h, :].astype(np.float64)
        for ai, a in enumerate(tiles):
            Q = q[rows_of[a], h, :].astype(np.float64)
            if Q.shape[0] == 0:
                continue
            s = (Q @ K.T) / np.sqrt(D)
            s -= s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            colmax = p.max(axis=0)                          # max over the tile's query rows
            np.maximum.at(out[hi, ai], tile_of_key, colmax)
    return out


def teacher_distribution(T):
    """Each query tile's row of T divided by its sum."""
    return T / T.sum(axis=-1, keepdims=True)


def recall(T, mask):
    """[H', n_q]: the teacher distribution's mass on the kept tiles; `mask`
    holds the matching rows of the block mask ([H', n_q, n_tiles] bool)."""
    return (teacher_distribution(T) * mask).sum(axis=-1)
