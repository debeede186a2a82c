"""Pins for the oracle's composition of one layer (veda_core.py, section
"one layer"): which spans a head group tiles and with which boxes, the
references-kept-whole branch, the column blocks and the per-head totals.
Expected values are derived by hand in tests/golden/layer_layouts.txt and
tests/golden/layer_totals.txt."""
import dataclasses
import os

import numpy as np
import pytest

from conftest import GOLDEN
from edge_cases import EDGE
from oracle import budget, layer, selection, tiles
import workloads


def _ranges(tokens):
    out = []
    for tok in tokens:
        if "-" in tok:
            a, b = tok.split("-")
            out.extend(range(int(a), int(b) + 1))
        else:
            out.append(int(tok))
    return out


def _golden_layouts():
    cases, cur = {}, None
    for line in open(os.path.join(GOLDEN, "layer_layouts.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        head, _, rest = line.partition(" ")
        if head == "case":
            name, seq = rest.split()
            cur = cases[name] = dict(seq_len=int(seq.split("=")[1]), spans=[], tiles={})
        elif head == "span":
            v = rest.split()
            cur["spans"].append((int(v[0]), tuple(int(x) for x in v[1:4]),
                                 tuple(int(x) for x in v[5:8])))
        elif head == "counts":
            cur["counts"] = tuple(int(x) for x in rest.split())
        elif head == "tile":
            idx, _, body = rest.partition(":")
            cur["tiles"][int(idx)] = _ranges(body.split())
    return cases


LAYOUTS = _golden_layouts()
# golden case -> (workload, target box of the head group or None for least padding)
_CASE_GROUP = {
    "ragged_refs_1x8x16": ("ragged_refs", (1, 8, 16)),
    "ragged_refs_least": ("ragged_refs", None),
    "refs_whole": ("refs_whole", None),
}


@pytest.mark.parametrize("case", sorted(LAYOUTS))
def test_group_layout_matches_hand_derivation(case):
    want = LAYOUTS[case]
    wname, shape = _CASE_GROUP[case]
    wl = EDGE[wname]
    assert wl.seq_len == want["seq_len"]
    gen, ref = budget.from_request(wl.generated), budget.from_request(wl.reference)
    # the group's box comes from layer.head_groups, as run() takes it
    groups = dict((tuple(heads), s) for s, heads in layer.head_groups(wl.head_shapes, wl.target[1]))
    heads = [h for h, s in enumerate(wl.head_shapes) if s == shape]
    box = groups[tuple(heads)]
    lay = layer.layout_for(wl, box, gen, ref)
    assert [tuple(s) for s in lay.shapes] == [s[2] for s in want["spans"]]
    assert (lay.n_ref, lay.n_video, lay.n_global, lay.n_tiles, lay.ref_tokens,
            lay.target_tokens) == want["counts"]
    for a, rows in want["tiles"].items():
        assert lay.tile_rows(a).tolist() == rows, f"tile {a}"
        assert lay.valid_count[a] == len(rows)


def test_head_groups_of_ragged_refs():
    wl = EDGE["ragged_refs"]
    got = layer.head_groups(wl.head_shapes, wl.target[1])
    assert got == [((2, 4, 16), [0, 2]), ((1, 8, 16), [1])]


def test_refs_whole_branch_makes_reference_rows_global():
    """A reference budget that keeps everything leaves the references untiled
    (their rows become global, ascending, after the video tiles) and leaves
    one column block; a budget that does not keep everything tiles them and
    gives them a block of their own."""
    wl = EDGE["refs_whole"]
    gen = budget.from_request(wl.generated)
    whole = budget.from_request(wl.reference)
    assert budget.keeps_all(whole)
    lay = layer.layout_for(wl, tiles.least_padding_shape(wl.target[1]), gen, whole)
    assert lay.n_ref == 0
    glob = lay.perm[lay.n_video * 128:]
    glob = glob[glob >= 0]
    assert glob.tolist() == list(range(0, 130)) + list(range(1330, 1500))
    blocks = selection.column_blocks(lay, gen, whole)
    assert [(b[0], b[1]) for b in blocks] == [(0, 18)]
    # Tiled, the (2,5,12) reference needs two tiles: no box fits inside it, a
    # single tile would need t >= 2, h >= 8, w >= 16 (256 cells), and of the
    # two-tile boxes (2,8,8) has the least aspect (4; (2,4,16) has 8,
    # (1,8,16) 16).
    tiled = layer.layout_for(wl, tiles.least_padding_shape(wl.target[1]), gen, (0.5, None))
    assert tiled.shapes[0] == (2, 8, 8)
    assert tiled.n_ref == 2 and tiled.n_video == 20
    assert [(b[0], b[1], b[2]) for b in selection.column_blocks(tiled, gen, (0.5, None))] == \
        [(0, 2, (0.5, None)), (2, 20, gen)]


def _golden_totals():
    out = []
    for line in open(os.path.join(GOLDEN, "layer_totals.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        left, right = line.split("->")
        name, group = left.split()
        out.append((name, group, tuple(int(x) for x in right.split())))
    return out


def _reduced(name):
    """The workload's geometry and budgets with few, narrow heads (the totals
    do not depend on the values), one head per distinct tile box."""
    wl = workloads.get(name)
    shapes = list(dict.fromkeys(wl.head_shapes))
    return dataclasses.replace(wl, n_heads=len(shapes), head_dim=64, dtype="f32",
                               head_shapes=tuple(shapes), bias=False)


@pytest.mark.parametrize("name,group,want", _golden_totals(),
                         ids=lambda x: x if isinstance(x, str) else "")
def test_layer_totals_match_hand_derivation(name, group, want):
    wl = _reduced(name)
    inp = workloads.generate(wl)
    groups, _ = layer.run(inp, do_attend=False)
    n_ref, n_video, n_global, n_tiles, kept, entries = want
    box = None if group == "least" else tuple(int(x) for x in group.split("x"))
    g = [g for g in groups if box is None or g.shape == box]
    assert len(g) == 1
    g = g[0]
    lay = g.layout
    assert (lay.n_ref, lay.n_video, lay.n_global, lay.n_tiles) == (n_ref, n_video, n_global, n_tiles)
    assert (g.kept.sum(axis=(1, 2)) == kept).all()
    assert (g.mask.sum(axis=(1, 2)) == entries).all()
    # every row keeps k_lo + extra(r) per block, whatever the scores
    for start, stop, keep_all, lo, hi, frac in selection.block_params(lay, g.blocks):
        per_row = g.kept[:, :, start:stop].sum(axis=2)
        want_row = lo + budget.bresenham(lay.n_video, frac).astype(np.int64)
        assert (per_row == want_row[None, :]).all()
    # the run's receipt counts: work = tile-list entries, dense = (S/128)^2 per head
    assert g.stats["work"] == entries * len(g.heads)
    assert g.stats["dense"] == len(g.heads) * (wl.seq_len / 128) ** 2
