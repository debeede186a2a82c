"""Keep budgets (oracle; test infrastructure only).

Follows `veda_core.py` (page 1), section "budgets": the (ratio, tiles)
record, sparsity_budget, keeps_all, _per_row, _split and _bresenham.
Python floats are IEEE doubles, so every step here is fp64.
"""
from __future__ import annotations

import math

import numpy as np

TILE = 128


def sparsity_budget(share):
    """Skipping `share` of the key tiles keeps ratio 1.0 - share (no tile
    count). 90% sparse is therefore 0.09999999999999998, not 0.1."""
    return (1.0 - float(share), None)


def from_request(req):
    """A workload's budget request ('sparsity'|'ratio'|'tiles', value) as the
    pages' (ratio, tiles) record."""
    kind, value = req
    if kind == "sparsity":
        return sparsity_budget(value)
    if kind == "ratio":
        return (float(value), None)
    if kind == "tiles":
        return (None, float(value))
    raise ValueError(kind)


def keeps_all(budget):
    """A ratio budget of at least 1 keeps every tile; a tile budget never
    counts as keep-all here (its split decides)."""
    return budget[1] is None and budget[0] >= 1.0


def per_row(budget, real_tokens, n_cols):
    """Per-query-row budget of one column block.

    A tile budget is used as is. A ratio budget is priced at equal cost: it
    is ratio times the square of the unpadded tile count, shared over the
    block's (possibly padded) column count, evaluated left to right as
    ((ratio * ideal) * ideal) / n_cols in doubles.
    """
    if budget[1] is not None:
        return float(budget[1])
    ideal = math.ceil(real_tokens / TILE)
    return budget[0] * ideal * ideal / n_cols


def split(b, n_cols):
    """(k_lo, k_hi, frac) for a per-row budget b over a block of n_cols key
    tiles (veda_core.py § budgets, _split), with 1 <= k_lo <= k_hi <= n_cols.

    A budget of n_cols or more keeps the whole block, (n, n, 0). Otherwise a
    row keeps the whole part of b, at least one tile and at most n_cols, and
    one tile more on the rows the Bresenham pattern picks; that pattern runs
    on the leftover b - k_lo, clipped to [0, 1] and rounded to 12 decimal
    places with Python's correctly rounded round().
    """
    if b >= n_cols:
        return n_cols, n_cols, 0.0
    k_lo = int(math.floor(b))
    if k_lo < 1:
        k_lo = 1
    if k_lo > n_cols:
        k_lo = n_cols
    k_hi = k_lo + 1 if k_lo < n_cols else n_cols
    leftover = b - k_lo
    if leftover < 0.0:
        leftover = 0.0
    if leftover > 1.0:
        leftover = 1.0
    return k_lo, k_hi, round(leftover, 12)


def bresenham(n_rows, frac):
    """extra[r] = floor((r+1) * frac) > floor(r * frac), r in [0, n_rows), in
    fp64: spreads floor(n_rows * frac) extra tiles evenly over the rows."""
    ramp = np.floor(np.arange(n_rows + 1, dtype=np.float64) * float(frac))
    return ramp[1:] > ramp[:-1]
