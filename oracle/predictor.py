"""Triplet pooling and tile-pair logits (oracle; test infrastructure only).

Follows `veda_core.py` (page 1), section "predictor": pool() and logits().
fp64 throughout. The pages use fp32 with an unstated reduction order; fp64 on
both sides lets the top-k decisions agree bit for bit.
"""
from __future__ import annotations

import math

import numpy as np


def pool(x, layout, heads):
    """[H', n_video, 3D] fp64: per head and video tile, [mean | max | min] of
    the tile's real rows (veda_core.py § predictor, pool).

    Padding slots never enter the max or the min (zero padding is a legal
    value, so it must not win). mean is the fp64 sum over the real rows
    divided by their count. A tile with no real row gets zeros.
    `x` is [S, H, D]; `heads` lists the head indices of the group.
    """
    nv = layout.n_video
    D = x.shape[2]
    heads = np.asarray(heads)
    out = np.zeros((len(heads), nv, 3 * D), dtype=np.float64)
    for a in range(nv):
        rows = layout.tile_rows(a)
        if rows.size == 0:
            continue
        X = x[rows][:, heads, :].astype(np.float64)          # [count, H', D]
        out[:, a, :D] = X.sum(axis=0) / rows.size
        out[:, a, D:2 * D] = X.max(axis=0)
        out[:, a, 2 * D:] = X.min(axis=0)
    return out


def logits(fq, fk, pq, pk):
    """[H', n_q, n_k] fp64 tile logits (veda_core.py § predictor, logits).

    Each pooled tile is projected per head, x_hat = f @ P + mean (the mean
    part of f is added back as a residual), and the logit of a tile pair is
    q_hat . k_hat / sqrt(D), D being the projection's output width.
    """
    D = pq.shape[-1]
    pq = np.asarray(pq, dtype=np.float64)
    pk = np.asarray(pk, dtype=np.float64)
    qh = np.matmul(fq, pq) + fq[..., :D]
    kh = np.matmul(fk, pk) + fk[..., :D]
    return np.matmul(qh, np.swapaxes(kh, 1, 2)) / math.sqrt(D)
