"""Tile plans and predictor projections (oracle; test infrastructure only).

Follows `veda_core.py` (page 1), section "tile plans and the predictor file":
choose_plan, head_groups, describe_grid and the float8 projections scaled
per head in load_bundle. Written from the rules, sharing nothing with the
product's reader.
"""
from __future__ import annotations

import math

import numpy as np


def plan_candidates(plans):
    """[(name, grid, shapes, head_shape)]: the plans in order, then each
    one's H <-> W mirror (grid (T, W, H), boxes (t, w, h), name + '_T')."""
    out = [(n, tuple(g), [tuple(s) for s in sh], hs) for n, g, sh, hs in plans]
    for n, g, sh, hs in plans:
        out.append((n + "_T", (g[0], g[2], g[1]), [(s[0], s[2], s[1]) for s in sh], hs))
    return out


def tiles_over(grid, box):
    """Tiles a grid needs with one box (each axis padded up)."""
    return math.prod(-(-g // b) for g, b in zip(grid, box))


def choose_plan(plans, grid):
    """(name, grid, exact): the candidate minimising (|log aspect - log
    video aspect| rounded to 3 places, |T - video T|, total tiles of its
    boxes on the video grid), the first one on a full tie; aspect = W / H."""
    grid = tuple(int(x) for x in grid)
    target = math.log(grid[2] / grid[1])
    cands = plan_candidates(plans)
    keys = [(round(abs(math.log(g[2] / g[1]) - target), 3), abs(g[0] - grid[0]),
             sum(tiles_over(grid, s) for s in sh)) for _, g, sh, _ in cands]
    best = min(range(len(cands)), key=lambda i: (keys[i], i))
    name, g, _, _ = cands[best]
    return name, g, g == grid


def head_groups(shapes, head_shape_row):
    """[(box, [heads])] for one layer: heads sharing a box, boxes in index order."""
    used = sorted(set(head_shape_row))
    return [(tuple(shapes[i]), [h for h, j in enumerate(head_shape_row) if j == i])
            for i in used]


def describe_grid(grid):
    """'<W*32>x<H*32>, <seconds> s': 32 pixels per latent cell; a latent
    length T >= 2 holds 17 * floor((T - 2) / 5) + 5 frames (T < 2: one),
    shown in seconds at 24 frames per second with one decimal."""
    T, H, W = grid
    frames = 1 if T < 2 else 17 * ((T - 2) // 5) + 5
    return f"{W * 32}x{H * 32}, {frames / 24:.1f} s"


def e4m3_value(code):
    """float64 value of float8 e4m3fn codes (uint8): 1 sign, 4 exponent bits
    (bias 7), 3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); the
    all-ones pattern (exponent 15, mantissa 7) is NaN and there is no
    infinity."""
    code = np.asarray(code, dtype=np.uint8)
    sign = np.where(code & 0x80, -1.0, 1.0)
    e = (code >> 3) & 0xF
    m = (code & 0x7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def to_bf16(x32):
    """float32 -> nearest bfloat16 (ties to even), as float32."""
    b = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return r.astype(np.uint32).view(np.float32)


def dequantize(codes, scale):
    """Projections stored as float8 with a per-head scale: the float32
    product code value x scale[head] (heads on axis 0), rounded to bf16."""
    v = e4m3_value(codes).astype(np.float32)
    return to_bf16(v * np.asarray(scale, dtype=np.float32).reshape(-1, 1, 1))
