"""Tile-masked attention with int8 q.k products (oracle; test infrastructure
only).

The news pages name Veda's own kernel an INT8 Triton kernel and say its
result is approximate, not exact arithmetic (comfyui-wiki Veda news,
"Rendimiento" / "Performances"; the Vflash guide's note on the kernel); they
print no quantisation scheme. Reading, the plainest symmetric scheme those
words and the tile structure support:

  key tile j of head h   s_k = max |k_r| over the tile's real rows r and all
                         of D, divided by 127; codes c_k = rint(k / s_k)
  query row i of head h  s_q = max |q_i| over D, divided by 127;
                         codes c_q = rint(q_i / s_q)
  logit(i, r)            (c_q . c_k) * s_q * s_k * D^-1/2
  then                   exactly attend(): softmax over the kept tiles' real
                         key rows, P V, output at the query's original row.

rint rounds half to even; codes lie in [-127, 127]; an all-zero row or tile
has scale 0, codes 0 and logits exactly 0. The codes are integers decided by
floating point, so they are decided in the precision the device takes them
in, fp32: inv = fp32(127 / amax), code = rint(fp32(x * inv)), scale =
fp32(amax / 127) (with amax = 0: inv = 0, scale = 0). The code dot products
are exact integers; everything after them is fp64.
"""
from __future__ import annotations

import numpy as np

from .attention import _softmax_rows

_F127 = np.float32(127.0)


def quantize(x):
    """Symmetric int8 codes of the fp32 values x as one group: (codes, scale)
    with codes an int8 array of x's shape and scale an fp32 scalar (above)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.abs(x).max()) if x.size else np.float32(0.0)
    if amax > 0:
        inv = np.float32(_F127 / amax)
        scale = np.float32(amax / _F127)
    else:
        inv = scale = np.float32(0.0)
    codes = np.clip(np.rint(np.float32(x * inv)), -127, 127).astype(np.int8)
    return codes, scale


def quantize_rows(x):
    """Codes and scales of each row of x [n, D] as its own group: (int8
    [n, D], fp32 [n])."""
    x = np.asarray(x, dtype=np.float32)
    codes = np.zeros(x.shape, dtype=np.int8)
    scales = np.zeros(x.shape[0], dtype=np.float32)
    for i in range(x.shape[0]):
        codes[i], scales[i] = quantize(x[i])
    return codes, scales


def key_tile_codes(k, layout, h, j):
    """The codes of key tile j of head h in tile order: int8 [128, D], rows
    past the tile's real rows zero, and the tile's fp32 scale."""
    D = k.shape[2]
    rows = layout.tile_rows(j)
    codes = np.zeros((128, D), dtype=np.int8)
    c, s = quantize(k[rows, h, :])
    codes[:len(rows)] = c
    return codes, s


def attend(q, k, v, layout, mask, heads, query_tiles=None, out=None):
    """attention.attend with the logits above (same arguments, same output:
    fp64 [S, H', D], every real row of the computed query tiles written)."""
    S, _, D = q.shape
    scale = D ** -0.5
    heads = np.asarray(heads)
    if out is None:
        out = np.zeros((S, len(heads), D), dtype=np.float64)
    tiles = range(layout.n_tiles) if query_tiles is None else query_tiles
    rows_of = [layout.tile_rows(j) for j in range(layout.n_tiles)]
    for hi, h in enumerate(heads):
        tile_codes = {}
        for a in tiles:
            qrows = rows_of[a]
            if qrows.size == 0:
                continue
            cols = np.nonzero(mask[hi, a])[0]
            if cols.size == 0:
                out[qrows, hi, :] = 0.0
                continue
            cq, sq = quantize_rows(q[qrows, h, :])
            logits, values = [], []
            for j in cols:
                if j not in tile_codes:
                    tile_codes[j] = key_tile_codes(k, layout, h, j)
                ck, sk = tile_codes[j]
                n = len(rows_of[j])
                dots = cq.astype(np.int64) @ ck[:n].astype(np.int64).T     # exact integers
                logits.append(dots.astype(np.float64) * sq.astype(np.float64)[:, None]
                              * np.float64(sk) * scale)
                values.append(v[rows_of[j], h, :].astype(np.float64))
            P = _softmax_rows(np.concatenate(logits, axis=1))
            out[qrows, hi, :] = P @ np.concatenate(values, axis=0)
    return out
