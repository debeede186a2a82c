"""Masked attention over the packed layout (oracle; test infrastructure only).

`attend` follows `veda_core.py` (page 1), reference_attend, which the page
names as the exact ground truth of the tile-skip kernel: softmax of
q.k * D^-1/2 over the key slots whose tile is kept for the query's tile and
that hold a real row; padding query slots produce nothing. Results go back to
the query's original row (scatter_).

`dense_attention` and `token_masked_attention` are textbook attention in the
original row order; they exist only to pin `attend` (keep-all budgets and
token-level masks must agree with it).
"""
from __future__ import annotations

import numpy as np


def _softmax_rows(s):
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def attend(q, k, v, layout, mask, heads, query_tiles=None, out=None):
    """Exact tile-masked attention, fp64.

    q, k, v    : [S, H, D] (any float dtype; promoted to fp64)
    mask       : [H', n_tiles, n_tiles] bool block mask, rows = query tiles
    heads      : the H' head indices the mask's first axis refers to
    query_tiles: optional subset of query tiles to compute (sampling)
    out        : optional [S, H', D] fp64 array to fill; allocated if None

    Returns out with every real row of the computed query tiles written at
    its original row index.
    """
    S, _, D = q.shape
    scale = D ** -0.5
    heads = np.asarray(heads)
    if out is None:
        out = np.zeros((S, len(heads), D), dtype=np.float64)
    tiles = range(layout.n_tiles) if query_tiles is None else query_tiles
    rows_of = [layout.tile_rows(j) for j in range(layout.n_tiles)]
    for hi, h in enumerate(heads):
        for a in tiles:
            qrows = rows_of[a]
            if qrows.size == 0:
                continue
            cols = np.nonzero(mask[hi, a])[0]
            krows = np.concatenate([rows_of[j] for j in cols]) if cols.size else \
                np.zeros(0, dtype=np.int64)
            if krows.size == 0:
                out[qrows, hi, :] = 0.0             # nothing to attend: zeros
                continue
            Q = q[qrows, h, :].astype(np.float64)
            K = k[krows, h, :].astype(np.float64)
            V = v[krows, h, :].astype(np.float64)
            P = _softmax_rows((Q @ K.T) * scale)
            out[qrows, hi, :] = P @ V
    return out


def dense_attention(q, k, v, h):
    """softmax(Q K^T / sqrt(D)) V for head h over all S rows, fp64 (textbook)."""
    D = q.shape[2]
    Q = q[:, h, :].astype(np.float64)
    K = k[:, h, :].astype(np.float64)
    V = v[:, h, :].astype(np.float64)
    return _softmax_rows((Q @ K.T) / np.sqrt(D)) @ V


def token_masked_attention(q, k, v, h, allowed):
    """Dense attention for head h where allowed[i, j] (original row order)
    says whether row i may attend row j; masked logits are -inf."""
    D = q.shape[2]
    Q = q[:, h, :].astype(np.float64)
    K = k[:, h, :].astype(np.float64)
    V = v[:, h, :].astype(np.float64)
    s = (Q @ K.T) / np.sqrt(D)
    s = np.where(allowed, s, -np.inf)
    return _softmax_rows(s) @ V
