"""Pins for the oracle's selection, mask and tile lists (veda_core.py,
section "selection")."""
import itertools

import numpy as np
import pytest

from oracle import selection, tiles, budget, layer
import workloads


def _brute_force_kept(s_row, allowed):
    """Keep column j iff fewer than `allowed` columns outrank it, where j'
    outranks j when s[j'] > s[j], or s[j'] == s[j] and j' < j; -inf never kept."""
    n = len(s_row)
    out = np.zeros(n, dtype=bool)
    for j in range(n):
        rank = sum(1 for jj in range(n)
                   if s_row[jj] > s_row[j] or (s_row[jj] == s_row[j] and jj < j))
        out[j] = rank < allowed and s_row[j] > -np.inf
    return out


def _tiny_layout(n_tiles):
    # n_tiles full tiles of (1,8,16) along w
    return tiles.build_layout([(0, (1, 8, 16 * n_tiles), (1, 8, 16))], 128 * n_tiles)


@pytest.mark.parametrize("seed", range(6))
def test_select_matches_brute_force_rank(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(3, 12))
    lay = _tiny_layout(n)
    H = 3
    # coarse values force many exact ties
    scores = rng.integers(-3, 4, size=(H, n, n)).astype(np.float64)
    scores[0] = rng.standard_normal((n, n))
    ratio = float(rng.uniform(0.05, 0.9))
    bud = (ratio, None)
    blocks = [(0, n, bud, lay.target_tokens)]
    kept = selection.select(scores, lay, blocks)
    (_, _, _, lo, hi, frac), = selection.block_params(lay, blocks)
    extra = budget.bresenham(n, frac)
    for h in range(H):
        for r in range(n):
            s = scores[h, r].copy()
            s[r] = np.inf                               # own tile
            want = _brute_force_kept(s, min(lo + int(extra[r]), hi))
            assert np.array_equal(kept[h, r], want), (h, r)


def test_select_two_blocks_own_tile_only_in_its_block():
    # ref block of 3 tiles, target block of 5: own tile forced only in the
    # block that holds the row; per-row counts lo+extra per block
    spans = [(0, (1, 8, 48), (1, 8, 16)), (384, (1, 8, 80), (1, 8, 16))]
    lay = tiles.build_layout(spans, 384 + 640)
    assert (lay.n_ref, lay.n_video) == (3, 8)
    rng = np.random.default_rng(11)
    scores = rng.standard_normal((2, 8, 8))
    gen, ref = (None, 2.0), (None, 1.0)
    blocks = selection.column_blocks(lay, gen, ref)
    kept = selection.select(scores, lay, blocks)
    for h in range(2):
        for r in range(8):
            assert kept[h, r, :3].sum() == 1 and kept[h, r, 3:].sum() == 2
            if r < 3:
                assert kept[h, r, r]                      # own tile in ref block
                assert kept[h, r, 3 + np.argmax(scores[h, r, 3:])]
            else:
                assert kept[h, r, r]
                assert kept[h, r, np.argmax(scores[h, r, :3])]


def test_select_keep_all_and_big_tile_budget():
    lay = _tiny_layout(5)
    scores = np.random.default_rng(0).standard_normal((2, 5, 5))
    for bud in [(1.0, None), (2.0, None), (None, 5.0), (None, 99.0)]:
        kept = selection.select(scores, lay, [(0, 5, bud, lay.target_tokens)])
        assert kept.all()


@pytest.mark.parametrize("name,per_head", [("tiny", 16), ("padding", 25), ("mid", 5017)])
def test_kept_totals_closed_form(name, per_head):
    """One column block: per head, lo*nv + floor(nv*frac) tiles are kept, which
    equals floor(ratio * ideal^2) (tiles budget: tiles * nv)."""
    inp = workloads.generate(name)
    groups, _ = layer.run(inp, do_attend=False)
    for g in groups:
        assert (g.kept.sum(axis=(1, 2)) == per_head).all()
        nv = g.layout.n_video
        assert g.kept[:, np.arange(nv), np.arange(nv)].all()      # own tile


def test_mask_global_rows_and_columns_dense():
    inp = workloads.generate("padding")
    groups, _ = layer.run(inp, do_attend=False)
    g = groups[0]
    lay, mask = g.layout, g.mask
    nv, n = lay.n_video, lay.n_tiles
    assert mask[:, :, nv:].all() and mask[:, nv:, :].all()
    assert np.array_equal(mask[:, :nv, :nv], g.kept)
    assert mask.sum() == g.stats["work"]                          # 248 per the closed form
    off, cols = selection.tile_lists(mask)
    for h in range(mask.shape[0]):
        for a in range(n):
            row = cols[h][off[h, a]:off[h, a + 1]]
            assert np.all(np.diff(row) > 0)
            assert np.array_equal(row, np.nonzero(mask[h, a])[0])


def test_row_counts_closed_form_offsets():
    """CSR offsets of video row r equal sum over blocks of r*lo + floor(r*frac)
    plus r*n_global; global rows add n_tiles each (every tile non-empty)."""
    inp = workloads.generate("padding")
    groups, _ = layer.run(inp, do_attend=False)
    g = groups[0]
    lay = g.layout
    off, _ = selection.tile_lists(g.mask)
    params = selection.block_params(lay, g.blocks)
    nv = lay.n_video
    for r in range(lay.n_tiles + 1):
        rv = min(r, nv)
        want = sum(rv * lo + int(np.floor(rv * frac)) for (_, _, _, lo, _, frac) in params)
        want += rv * lay.n_global + max(0, r - nv) * lay.n_tiles
        assert (off[:, r] == want).all()
