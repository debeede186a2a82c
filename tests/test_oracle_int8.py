"""Pins for the oracle's int8 q.k attention (oracle/int8.py): the quantiser
against its defining properties and hand-worked codes, and the attention
against the exact oracle where the quantisation is lossless or undone."""
import numpy as np
import pytest

import workloads
from oracle import attention, int8, layer, tiles


def test_codes_are_symmetric_absmax_int8():
    """Codes lie in [-127, 127], the largest |x| maps to +-127 with x's sign,
    and code * scale is within half a step of x (rounding to the nearest
    code; the fp32 reciprocal adds at most a few ulps)."""
    rng = np.random.default_rng(5)
    for n in (1, 7, 128):
        x = workloads.bf16_round(rng.standard_normal((40, n)).astype(np.float32) * 3)
        codes, scales = int8.quantize_rows(x)
        assert codes.dtype == np.int8 and np.abs(codes.astype(int)).max() <= 127
        for i in range(x.shape[0]):
            j = np.argmax(np.abs(x[i]))
            assert codes[i, j] == (127 if x[i, j] > 0 else -127)
            assert scales[i] == np.float32(np.abs(x[i]).max() / np.float32(127))
            err = np.abs(codes[i].astype(np.float64) * scales[i] - x[i])
            assert err.max() <= scales[i] * (0.5 + 1e-5)


def test_hand_worked_codes_round_half_to_even():
    """Row (127, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5) * 2^-3: the scale is
    exactly 2^-3, every other value sits halfway between two codes, and
    rounding half to even gives 0, 2, 2, 0, -2, -2, 126."""
    x = np.array([127, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5], dtype=np.float32) / 8
    codes, scale = int8.quantize(x)
    assert scale == np.float32(0.125)
    assert codes.tolist() == [127, 0, 2, 2, 0, -2, -2, 126]


def test_zero_group_has_zero_scale_and_codes():
    codes, scale = int8.quantize(np.zeros(16, dtype=np.float32))
    assert scale == 0 and not codes.any()


def _layout():
    # 5 x 12 x 20 grid in (4, 4, 8) boxes (18 ragged tiles) and 64 text rows
    return tiles.build_layout([(0, (5, 12, 20), (4, 4, 8))], 1264)


def _lossless(shape, rng, scale_of_row):
    """Integers in [-127, 127] whose first column is 127, times a power of
    two per row: every group (row or tile) quantises without loss."""
    n = rng.integers(-127, 128, size=shape)
    n[..., 0] = 127
    return n.astype(np.float32) * scale_of_row


def test_lossless_inputs_reach_exact_attention():
    """When every query row and every key tile is an integer multiple of a
    power of two with its absmax at 127 steps, the codes are those integers
    and the int8 logits equal the exact ones, so the int8 attention equals
    the exact oracle. Steps differ per query row and per key tile, so a
    scale taken over the wrong group (the whole head, a row of K, padding
    included or not) breaks the equality."""
    rng = np.random.default_rng(11)
    lay = _layout()
    S, H, D = lay.seq_len, 2, 16
    row_step = np.float32(2.0) ** -rng.integers(2, 6, size=(S, H, 1)).astype(np.float32)
    q = _lossless((S, H, D), rng, row_step)
    k = np.zeros((S, H, D), dtype=np.float32)
    for j in range(lay.n_tiles):
        rows = lay.tile_rows(j)
        for h in range(H):
            step = np.float32(2.0) ** -float(rng.integers(2, 6))
            k[rows, h] = _lossless((len(rows), D), rng, step)
    v = rng.standard_normal((S, H, D))
    mask = rng.random((H, lay.n_tiles, lay.n_tiles)) < 0.4
    mask |= np.eye(lay.n_tiles, dtype=bool)[None]
    want = attention.attend(q, k, v, lay, mask, [0, 1])
    got = int8.attend(q, k, v, lay, mask, [0, 1])
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_equals_exact_attention_on_dequantised_inputs():
    """On any inputs the int8 logits are the exact logits of the dequantised
    tensors (query rows code * s_q, key tiles code * s_k): the int8 oracle
    equals the exact oracle fed those tensors."""
    inp = workloads.generate("padding")
    groups, _ = layer.run(inp, do_attend=False)
    g = groups[0]
    lay = g.layout
    qd = np.zeros_like(inp.q, dtype=np.float64)
    kd = np.zeros_like(inp.k, dtype=np.float64)
    for h in range(inp.q.shape[1]):
        for j in range(lay.n_tiles):
            rows = lay.tile_rows(j)
            cq, sq = int8.quantize_rows(inp.q[rows, h])
            qd[rows, h] = cq * sq.astype(np.float64)[:, None]
            ck, sk = int8.key_tile_codes(inp.k, lay, h, j)
            kd[rows, h] = ck[:len(rows)] * np.float64(sk)
        # rows no tile holds keep zeros: attend reads only real rows
    tiles_sel = np.arange(0, lay.n_tiles, 3)
    want = attention.attend(qd, kd, inp.v, lay, g.mask, g.heads, query_tiles=tiles_sel)
    got = int8.attend(inp.q, inp.k, inp.v, lay, g.mask, g.heads, query_tiles=tiles_sel)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_zero_query_row_averages_the_kept_values():
    """A query row of zeros has logits 0 against every key: its output is the
    plain mean of the kept keys' values."""
    rng = np.random.default_rng(3)
    lay = _layout()
    S, D = lay.seq_len, 8
    q = rng.standard_normal((S, 1, D)).astype(np.float32)
    k = rng.standard_normal((S, 1, D)).astype(np.float32)
    v = rng.standard_normal((S, 1, D))
    a = 4
    r0 = lay.tile_rows(a)[0]
    q[r0] = 0.0
    mask = np.zeros((1, lay.n_tiles, lay.n_tiles), dtype=bool)
    mask[0, a, [1, 4, 9]] = True
    got = int8.attend(q, k, v, lay, mask, [0], query_tiles=[a])
    keys = np.concatenate([lay.tile_rows(j) for j in (1, 4, 9)])
    np.testing.assert_allclose(got[r0, 0], v[keys, 0].mean(axis=0), rtol=0, atol=1e-12)


def test_key_tile_codes_layout():
    """Codes come in tile order with the tile's real rows first and zero
    padding rows after them; the scale is the tile's own."""
    rng = np.random.default_rng(8)
    lay = _layout()
    k = rng.standard_normal((lay.seq_len, 1, 8)).astype(np.float32)
    ragged = [j for j in range(lay.n_tiles) if 0 < lay.valid_count[j] < 128]
    assert ragged
    j = ragged[0]
    rows = lay.tile_rows(j)
    codes, s = int8.key_tile_codes(k, lay, 0, j)
    assert codes.shape == (128, 8) and not codes[len(rows):].any()
    c2, s2 = int8.quantize(k[rows, 0])
    assert s == s2 and np.array_equal(codes[:len(rows)], c2)


@pytest.mark.parametrize("name", ["padding", "ragged_refs"])
def test_int8_error_against_exact_attention_is_bounded(name):
    """On the synthetic bf16 workloads the int8 reading stays within max-abs
    5e-2 and mean-abs 2.5e-3 of exact attention (the tolerance the int8
    kernel is held to against the exact oracle)."""
    from edge_cases import EDGE
    wl = EDGE.get(name) or workloads.get(name)
    inp = workloads.generate(wl)
    groups, _ = layer.run(inp, do_attend=False)
    for g in groups:
        want = attention.attend(inp.q, inp.k, inp.v, g.layout, g.mask, g.heads)
        got = int8.attend(inp.q, inp.k, inp.v, g.layout, g.mask, g.heads)
        rows = np.concatenate([g.layout.tile_rows(a) for a in range(g.layout.n_tiles)])
        err = np.abs(got[rows] - want[rows])
        assert err.max() <= 5e-2 and err.mean() <= 2.5e-3
