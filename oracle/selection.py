"""Head-aware top-k tile selection and the block mask (oracle; test
infrastructure only).

Follows `veda_core.py` (page 1), section "selection": column_blocks,
select, block_mask and tile_index_list.
"""
from __future__ import annotations

import numpy as np

from .budget import keeps_all, per_row, split, bresenham


def column_blocks(layout, generated, reference):
    """[(start, stop, budget, real_tokens)] (veda_core.py § selection,
    column_blocks): the key tiles split into independent top-k blocks. The
    target tiles always form one block under the generated budget; when the
    layout holds reference tiles they form a block of their own, first, under
    the reference budget, so that the target's neighbours cannot crowd the
    references out of a single shared top-k."""
    blocks = []
    if layout.n_ref > 0:
        blocks.append((0, layout.n_ref, reference, layout.ref_tokens))
    blocks.append((layout.n_ref, layout.n_video, generated, layout.target_tokens))
    return blocks


def block_params(layout, blocks):
    """Per block: (start, stop, keep_all, lo, hi, frac) as select() uses them."""
    out = []
    for start, stop, budget, real in blocks:
        n = stop - start
        if keeps_all(budget):
            out.append((start, stop, True, n, n, 0.0))
            continue
        lo, hi, frac = split(per_row(budget, real, n), n)
        out.append((start, stop, False, lo, hi, frac))
    return out


def select(scores, layout, blocks):
    """kept [H', n_video, n_video] bool (veda_core.py § selection, select).

    Per head, video row r and column block [start, stop):
      * empty key tiles score -inf (never kept);
      * when r lies inside the block, its own tile scores +inf (always kept,
        and it counts against the budget);
      * tiles are ranked by score, highest first; equal scores rank the lower
        column first (the pages leave ties to torch.topk; this is the reading
        taken);
      * the first k_lo + extra[r] ranked tiles are kept, extra being the
        Bresenham pattern over all n_video rows; -inf tiles are dropped.
    A ratio budget >= 1 keeps every non-empty tile of the block.
    """
    H, nv = scores.shape[0], layout.n_video
    kv_ok = layout.kv_ok
    kept = np.zeros((H, nv, nv), dtype=bool)
    rows = np.arange(nv)
    for (start, stop, budget, real), (_, _, keep_all, lo, hi, frac) in zip(
            blocks, block_params(layout, blocks)):
        n = stop - start
        if keep_all:
            kept[:, :, start:stop] = kv_ok[start:stop][None, None, :]
            continue
        s = np.array(scores[:, :, start:stop], dtype=np.float64, copy=True)
        s[:, :, ~kv_ok[start:stop]] = -np.inf
        inside = (rows >= start) & (rows < stop)
        s[:, rows[inside], rows[inside] - start] = np.inf
        extra = bresenham(nv, frac)
        allowed = lo + extra.astype(np.int64)                     # [nv]
        cols = np.broadcast_to(np.arange(n), s.shape)
        order = np.lexsort((cols, -s), axis=-1)                   # score desc, col asc
        ranked = np.take_along_axis(s, order, axis=-1)
        rank = np.arange(n)[None, None, :]
        keep_ranked = (rank < hi) & (rank < allowed[None, :, None]) & (ranked > -np.inf)
        blk = np.zeros((H, nv, n), dtype=bool)
        np.put_along_axis(blk, order, keep_ranked, axis=-1)
        kept[:, :, start:stop] = blk
    return kept


def block_mask(kept, layout):
    """[H', n_tiles, n_tiles] bool, rows = query tiles
    (veda_core.py § selection, block_mask): the video x video quadrant is the
    kept set; every row sees the non-empty global tiles; global rows see every
    non-empty tile."""
    H, n, nv = kept.shape[0], layout.n_tiles, layout.n_video
    kv_ok = layout.kv_ok
    mask = np.zeros((H, n, n), dtype=bool)
    mask[:, :nv, :nv] = kept
    mask[:, :, nv:] = kv_ok[nv:][None, None, :]
    mask[:, nv:, :] = kv_ok[None, None, :]
    return mask


def tile_lists(mask):
    """The mask as per-row ascending lists of kept tiles
    (veda_core.py § selection, tile_index_list), in CSR form per head:
    (offsets [H', n_tiles + 1] int64, cols [H'] list of int64 arrays)."""
    H, n, _ = mask.shape
    counts = mask.sum(axis=-1)
    offsets = np.zeros((H, n + 1), dtype=np.int64)
    offsets[:, 1:] = np.cumsum(counts, axis=-1)
    cols = [np.nonzero(mask[h].reshape(-1))[0] % n for h in range(H)]
    return offsets, cols
