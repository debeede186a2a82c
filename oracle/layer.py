"""One layer of Veda attention (oracle; test infrastructure only).

Follows `veda_core.py` (page 1), section "one layer", attention(): heads are
grouped by their target tile box; per group the layout is built (reference
spans tiled with their least-padding box unless the reference budget keeps
everything, in which case reference rows stay global), q and k are pooled,
tile pairs scored, top-k selected per column block, the block mask formed and
attention computed over it.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import tiles, budget, predictor, selection, attention


def head_groups(head_shapes, target_grid):
    """[(shape, [heads])] in order of first appearance; a None shape asks for
    the least-padding box of the target grid (veda_core.py § tile plans,
    head_groups, with the plan's shapes given per head)."""
    groups = {}
    for h, s in enumerate(head_shapes):
        s = tiles.least_padding_shape(target_grid) if s is None else tuple(s)
        groups.setdefault(s, []).append(h)
    return list(groups.items())


def layout_for(wl, shape, generated, reference):
    """Build the layout of one head group (the pages' cache key is the
    geometry, the shape and whether references are tiled)."""
    tile_refs = not budget.keeps_all(reference)
    spans = []
    if tile_refs:
        for start, g in wl.refs:
            spans.append((start, g, tiles.least_padding_shape(g)))
    spans.append((wl.target[0], wl.target[1], shape))
    return tiles.build_layout(spans, wl.seq_len)


@dataclass
class GroupResult:
    shape: tuple
    heads: list
    layout: object
    blocks: list
    scores: np.ndarray = None
    kept: np.ndarray = None
    mask: np.ndarray = None
    stats: dict = field(default_factory=dict)


def run(inp, attend_tiles="all", do_attend=True):
    """The whole layer for workloads.Inputs `inp`.

    attend_tiles: "all", or {group shape: array of query tiles} to compute
    attention for a sample only. Returns (groups, out) where out is
    [S, H, D] fp64 (rows of unsampled tiles stay 0).
    """
    wl = inp.workload
    generated = budget.from_request(wl.generated)
    reference = budget.from_request(wl.reference)
    S, H, D = inp.q.shape
    out = np.zeros((S, H, D), dtype=np.float64) if do_attend else None
    groups = []
    for shape, heads in head_groups(wl.head_shapes, wl.target[1]):
        lay = layout_for(wl, shape, generated, reference)
        blocks = selection.column_blocks(lay, generated, reference)
        fq = predictor.pool(inp.q, lay, heads)
        fk = predictor.pool(inp.k, lay, heads)
        scores = predictor.logits(fq, fk, inp.proj_q[heads], inp.proj_k[heads])
        kept = selection.select(scores, lay, blocks)
        mask = selection.block_mask(kept, lay)
        g = GroupResult(shape, heads, lay, blocks, scores, kept, mask)
        g.stats = dict(
            kept=int(kept.sum()),
            pairs=len(heads) * lay.n_video ** 2,
            work=int(kept.sum()) + len(heads) * lay.n_global * (lay.n_tiles + lay.n_video),
            dense=len(heads) * (S / 128) ** 2,
            mask_pairs=int(mask.sum()),
        )
        if do_attend:
            qt = None if attend_tiles == "all" else attend_tiles.get(shape)
            sub = attention.attend(inp.q, inp.k, inp.v, lay, mask, heads, query_tiles=qt)
            out[:, heads, :] += sub
        groups.append(g)
    return groups, out
