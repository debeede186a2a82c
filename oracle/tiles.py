"""Tile boxes and the packed layout (oracle; test infrastructure only).

Follows `veda_core.py` (page 1), section "tiles": functions shapes,
_padded/_count, least_padding_shape, span_tiles and build_layout.
Everything here is integer work written as literal loops.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

TILE = 128


class VedaError(ValueError):
    """A layout that cannot be used (veda_core.py, VedaError)."""


def shapes():
    """Every (t, h, w) of powers of two with t*h*w == 128, sorted as tuples.

    veda_core.py § tiles, shapes(): i, j range so that 2^i * 2^j divides 128.
    """
    out = []
    for i in range(8):
        for j in range(8 - i):
            out.append((2 ** i, 2 ** j, TILE // (2 ** i * 2 ** j)))
    return sorted(out)


def _ceil_div(a, b):
    return -(-a // b)


def tile_count(grid, shape):
    """Tiles needed for `grid` once every axis is padded up to a multiple of
    `shape` (veda_core.py § tiles, _padded and _count)."""
    n = 1
    for g, s in zip(grid, shape):
        n *= _ceil_div(g, s)
    return n


def least_padding_shape(grid):
    """Box that pads `grid` least; ties go to the smallest max/min aspect,
    then to the first tuple. Boxes that fit inside the grid on every axis are
    preferred; if none fits, all 36 are candidates
    (veda_core.py § tiles, least_padding_shape)."""
    all_shapes = shapes()
    fit = [s for s in all_shapes if all(a <= b for a, b in zip(s, grid))]
    cands = fit if fit else all_shapes
    best = None
    best_key = None
    for s in cands:
        key = (tile_count(grid, s), max(s) / min(s), s)
        if best_key is None or key < best_key:
            best, best_key = s, key
    return best


def span_tiles(start, grid, shape):
    """[n_tiles, 128] int64 row ids of one span, -1 on padding.

    veda_core.py § tiles, span_tiles: the grid is padded to a multiple of the
    box on every axis; boxes are visited with the h-box outermost, then the
    w-box, then the t-box innermost; inside a box the cells go t, h, w
    row-major; a cell's id is start + (t*H + h)*W + w when it lies inside the
    grid, else -1; finally the real ids of each tile are moved to its front
    in their order (a stable partition), so padding sits at the end.
    """
    T, H, W = grid
    st, sh, sw = shape
    nbt, nbh, nbw = _ceil_div(T, st), _ceil_div(H, sh), _ceil_div(W, sw)
    tiles = []
    for bh in range(nbh):
        for bw in range(nbw):
            for bt in range(nbt):
                cells = []
                for dt in range(st):
                    for dh in range(sh):
                        for dw in range(sw):
                            t, h, w = bt * st + dt, bh * sh + dh, bw * sw + dw
                            if t < T and h < H and w < W:
                                cells.append(start + (t * H + h) * W + w)
                            else:
                                cells.append(-1)
                real = [c for c in cells if c >= 0]
                pad = [c for c in cells if c < 0]
                tiles.append(real + pad)
    return np.array(tiles, dtype=np.int64).reshape(-1, TILE)


@dataclass
class Layout:
    """The packed sequence (veda_core.py § tiles, build_layout's record).

    perm[N]        : packed slot -> original row, -1 for padding
    valid_count[n] : real rows per tile
    """
    perm: np.ndarray
    valid_count: np.ndarray
    n_video: int
    n_ref: int
    n_global: int
    n_tiles: int
    ref_tokens: int
    target_tokens: int
    seq_len: int
    shapes: list

    @property
    def n_slots(self):
        return self.n_tiles * TILE

    @property
    def kv_ok(self):
        return self.valid_count > 0

    def tile_rows(self, a):
        """Original rows of tile a, real ones only, in slot order."""
        ids = self.perm[a * TILE:(a + 1) * TILE]
        return ids[ids >= 0]


def _check_spans(spans, seq_len):
    """Refuses span lists the packing cannot use (veda_core.py § tiles,
    build_layout): there must be a target span; spans come in packed order,
    each one beginning no earlier than where the previous one ended and lying
    inside [0, seq_len). Reading: a negative start is refused as well (the
    page tests only order, overlap and overrun)."""
    if len(spans) == 0:
        raise VedaError("no video span given: at least one span, the generated video, is required")
    prev_end = 0
    for start, grid, _ in spans:
        end = start + grid[0] * grid[1] * grid[2]
        if start < 0 or start < prev_end or end > seq_len:
            raise VedaError(f"video span [{start}, {end}) is out of packed order or "
                            f"outside the sequence of {seq_len} rows")
        prev_end = end


def build_layout(spans, seq_len):
    """One permutation of the packed sequence.

    veda_core.py § tiles, build_layout: `spans` = [(start, grid, shape)] in
    packed order with the target last. The tiles of each span come first, in
    span order (span_tiles). Every row that no span covers is a global row
    (text, audio, conditions kept whole); the global rows follow the video
    tiles in ascending row order, 128 to a tile, and the last global tile is
    padded with -1.
    """
    _check_spans(spans, seq_len)
    video = [span_tiles(start, grid, shape) for start, grid, shape in spans]
    n_video = sum(t.shape[0] for t in video)

    in_span = [False] * seq_len
    for start, grid, _ in spans:
        for r in range(start, start + grid[0] * grid[1] * grid[2]):
            in_span[r] = True
    global_rows = [r for r in range(seq_len) if not in_span[r]]
    n_global = _ceil_div(len(global_rows), TILE)
    global_slots = global_rows + [-1] * (n_global * TILE - len(global_rows))

    perm = np.array([r for t in video for r in t.reshape(-1)] + global_slots, dtype=np.int64)
    n_tiles = n_video + n_global
    valid = np.zeros(n_tiles, dtype=np.int64)
    for a in range(n_tiles):
        for slot in range(a * TILE, (a + 1) * TILE):
            if perm[slot] >= 0:
                valid[a] += 1

    def rows_of(sp):
        return sum(g[0] * g[1] * g[2] for _, g, _ in sp)

    return Layout(
        perm=perm, valid_count=valid, n_video=n_video,
        n_ref=n_video - video[-1].shape[0], n_global=n_global, n_tiles=n_tiles,
        ref_tokens=rows_of(spans[:-1]), target_tokens=rows_of(spans[-1:]),
        seq_len=seq_len, shapes=[s for _, _, s in spans],
    )
