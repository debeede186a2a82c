"""Pins for the oracle's tile boxes and layout (veda_core.py, section "tiles")."""
import os
import re

import numpy as np
import pytest

from conftest import GOLDEN
from oracle import tiles
from oracle.tiles import TILE, VedaError


def _golden_least_padding():
    out = []
    for line in open(os.path.join(GOLDEN, "least_padding.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        left, right = line.split("->")
        grid = tuple(int(x) for x in left.split())
        t, h, w, n = (int(x) for x in right.split())
        out.append((grid, (t, h, w), n))
    return out


def _golden_span_tiles():
    cases, cur = [], None
    for line in open(os.path.join(GOLDEN, "span_tiles.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        if line.startswith("case"):
            v = [int(x) for x in line.split()[1:]]
            cur = (v[0], tuple(v[1:4]), tuple(v[4:7]), [])
            cases.append(cur)
        else:
            body = line.split(":", 1)[1]
            ids = []
            for tok in body.split():
                if "-" in tok:
                    a, b = tok.split("-")
                    ids.extend(range(int(a), int(b) + 1))
                else:
                    ids.append(int(tok))
            cur[3].append(ids)
    return cases


def test_shapes_are_the_36_power_of_two_boxes():
    s = tiles.shapes()
    # 2^a * 2^b * 2^c = 2^7 has C(9, 2) = 36 solutions in non-negative integers
    assert len(s) == 36 and len(set(s)) == 36
    for t, h, w in s:
        assert t * h * w == TILE
        for x in (t, h, w):
            assert x & (x - 1) == 0
    assert s == sorted(s)
    assert s[0] == (1, 1, 128) and s[-1] == (128, 1, 1)


@pytest.mark.parametrize("grid,shape,n", _golden_least_padding())
def test_least_padding_hand_examples(grid, shape, n):
    assert tiles.least_padding_shape(grid) == shape
    assert tiles.tile_count(grid, shape) == n


def test_least_padding_falls_back_to_all_boxes():
    # a grid smaller than every box on some axis: (1,1,1) fits nothing -> the
    # choice is over all 36, each needing one tile; the most cubic wins, (4,4,8)
    assert tiles.least_padding_shape((1, 1, 1)) == (4, 4, 8)


@pytest.mark.parametrize("case", _golden_span_tiles(), ids=lambda c: f"{c[1]}-{c[2]}")
def test_span_tiles_hand_examples(case):
    start, grid, shape, want = case
    got = tiles.span_tiles(start, grid, shape)
    assert got.shape == (len(want), TILE)
    for i, ids in enumerate(want):
        real = got[i][got[i] >= 0].tolist()
        assert real == ids
        assert (got[i][len(ids):] == -1).all()


def _box_counts(grid, shape):
    """Real rows per box from the box's real extents: prod(min(s, g - b*s)).
    Box order: h-box outer, w-box, t-box inner."""
    (T, H, W), (st, sh, sw) = grid, shape
    nb = [-(-g // s) for g, s in zip(grid, shape)]
    out = []
    for bh in range(nb[1]):
        for bw in range(nb[2]):
            for bt in range(nb[0]):
                out.append(min(st, T - bt * st) * min(sh, H - bh * sh) * min(sw, W - bw * sw))
    return out


@pytest.mark.parametrize("grid,shape", [((5, 12, 20), (4, 4, 8)), ((3, 7, 9), (2, 2, 32)),
                                        ((31, 48, 70), (1, 16, 8)), ((1, 48, 84), (1, 16, 8)),
                                        ((9, 5, 13), (8, 4, 4)), ((2, 1, 300), (1, 1, 128))])
def test_span_tiles_bijection_counts_and_prefix(grid, shape):
    start = 17
    t = tiles.span_tiles(start, grid, shape)
    rows = grid[0] * grid[1] * grid[2]
    real = t[t >= 0]
    assert np.array_equal(np.sort(real), np.arange(start, start + rows))
    assert t.shape[0] == tiles.tile_count(grid, shape)
    counts = (t >= 0).sum(1)
    assert counts.tolist() == _box_counts(grid, shape)
    for row in t:                                 # real ids form a prefix
        c = int((row >= 0).sum())
        assert (row[:c] >= 0).all() and (row[c:] < 0).all()
    assert (counts > 0).all()                     # every box holds its origin cell


def test_build_layout_headline_geometry():
    spans = [(0, (1, 48, 84), (1, 16, 8)), (4032, (31, 48, 70), (1, 16, 8))]
    lay = tiles.build_layout(spans, 108448)
    assert (lay.n_tiles, lay.n_video, lay.n_ref, lay.n_global) == (872, 870, 33, 2)
    assert lay.n_slots == 111616
    real = lay.perm[lay.perm >= 0]
    assert np.array_equal(np.sort(real), np.arange(108448))
    vc = lay.valid_count
    assert ((vc > 0) & (vc < TILE)).sum() == 96
    assert (vc == 96).sum() == 93 and (vc == 64).sum() == 3
    # global rows: the 256 text rows, ascending, two full tiles
    assert np.array_equal(lay.perm[870 * TILE:], np.arange(108192, 108448))
    assert lay.ref_tokens == 4032 and lay.target_tokens == 104160


def test_build_layout_padding_geometry():
    lay = tiles.build_layout([(0, (5, 12, 20), (4, 4, 8))], 1264)
    assert (lay.n_tiles, lay.n_video, lay.n_global) == (19, 18, 1)
    assert lay.valid_count.tolist() == [128, 32, 128, 32, 64, 16] * 3 + [64]
    tail = lay.perm[18 * TILE:]
    assert np.array_equal(tail[:64], np.arange(1200, 1264)) and (tail[64:] == -1).all()


def test_build_layout_globals_between_spans():
    # rows 0-9 text, span 10..(10+64), rows 74-99 text, span 100..(100+128), rows 228-229 text
    spans = [(10, (1, 8, 8), (1, 8, 16)), (100, (2, 8, 8), (2, 8, 8))]
    lay = tiles.build_layout(spans, 230)
    assert lay.n_video == 2 and lay.n_global == 1 and lay.n_ref == 1
    g = lay.perm[2 * TILE:]
    want = list(range(0, 10)) + list(range(74, 100)) + [228, 229]
    assert g[:len(want)].tolist() == want and (g[len(want):] == -1).all()


@pytest.mark.parametrize("spans,seq", [
    ([], 10),
    ([(0, (1, 8, 8), (1, 8, 16)), (32, (1, 8, 8), (1, 8, 16))], 200),   # overlap
    ([(0, (1, 8, 8), (1, 8, 16))], 63),                                  # overrun
    ([(-1, (1, 8, 8), (1, 8, 16))], 100),                                # negative start
])
def test_build_layout_refuses(spans, seq):
    with pytest.raises(VedaError):
        tiles.build_layout(spans, seq)
