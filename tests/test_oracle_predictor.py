"""Pins for the oracle's pooling and logits (veda_core.py, section "predictor")."""
import math

import numpy as np
import pytest

from oracle import predictor, tiles
import workloads


def _grid_boxes(x, grid, shape):
    """Pool by reshaping the [T,H,W] grid into boxes (valid when the box
    divides the grid): an independent route to each tile's rows, in the box
    order h-box, w-box, t-box."""
    T, H, W = grid
    st, sh, sw = shape
    S, nh, D = x.shape
    g = x.reshape(T // st, st, H // sh, sh, W // sw, sw, nh, D)
    g = g.transpose(2, 4, 0, 1, 3, 5, 6, 7).reshape(-1, st * sh * sw, nh, D)
    return g


@pytest.mark.parametrize("grid,shape", [((4, 16, 16), (2, 8, 8)), ((8, 8, 8), (4, 4, 8)),
                                        ((2, 16, 32), (1, 8, 16))])
def test_pool_matches_box_reshape(grid, shape):
    rng = np.random.default_rng(3)
    S = grid[0] * grid[1] * grid[2]
    x = rng.standard_normal((S, 3, 16))
    lay = tiles.build_layout([(0, grid, shape)], S)
    f = predictor.pool(x, lay, [0, 1, 2])
    boxes = _grid_boxes(x, grid, shape)              # [n_tiles, 128, H, D]
    D = 16
    np.testing.assert_allclose(f[:, :, :D], boxes.mean(axis=1).transpose(1, 0, 2), rtol=0, atol=1e-14)
    assert np.array_equal(f[:, :, D:2 * D], boxes.max(axis=1).transpose(1, 0, 2))
    assert np.array_equal(f[:, :, 2 * D:], boxes.min(axis=1).transpose(1, 0, 2))


def test_pool_ignores_padding_slots():
    # (1,8,8) grid in a (1,8,16) box: 64 real rows, 64 padding slots. All real
    # values negative -> the max must be negative (a zero pad would win), and
    # the mean divides by 64, not 128.
    x = -1.0 - np.arange(64 * 2 * 4, dtype=np.float64).reshape(64, 2, 4) / 1000.0
    lay = tiles.build_layout([(0, (1, 8, 8), (1, 8, 16))], 64)
    f = predictor.pool(x, lay, [0, 1])
    assert (f[:, 0, 4:8] < 0).all()
    np.testing.assert_allclose(f[:, 0, :4], x.mean(axis=0), rtol=0, atol=1e-14)
    x2 = -x
    f2 = predictor.pool(x2, lay, [1])
    assert (f2[:, 0, 8:] > 0).all()                 # min of positive real rows stays positive
    assert np.array_equal(f2[0, 0, 8:], x2[:, 1, :].min(axis=0))


def test_logits_zero_projection_is_scaled_product_of_means():
    rng = np.random.default_rng(5)
    H, n, D = 2, 6, 8
    fq = rng.standard_normal((H, n, 3 * D))
    fk = rng.standard_normal((H, n, 3 * D))
    P = np.zeros((H, 3 * D, D))
    s = predictor.logits(fq, fk, P, P)
    for h in range(H):
        for i in range(n):
            for j in range(n):
                want = sum(fq[h, i, d] * fk[h, j, d] for d in range(D)) / math.sqrt(D)
                assert abs(s[h, i, j] - want) < 1e-12


def test_logits_embedding_identity_tiny():
    """Tiny workload: P_q = [W_q W_k^T - I; 0; 0], P_k = 0 gives
    score = (m_q W_q).(m_k W_k) / sqrt(D); a dropped residual, a transposed P or
    a wrong block of f breaks it."""
    inp = workloads.generate("tiny")
    wl = inp.workload
    lay = tiles.build_layout([(0, wl.target[1], (2, 8, 8))], wl.seq_len)
    heads = [0, 1]
    fq = predictor.pool(inp.q, lay, heads)
    fk = predictor.pool(inp.k, lay, heads)
    s = predictor.logits(fq, fk, inp.proj_q, inp.proj_k)
    D = wl.head_dim
    wq = inp.proj_q  # float32 values both sides use
    for h in heads:
        mq = fq[h, :, :D] @ inp.extras["w_q"][h]
        mk = fk[h, :, :D] @ inp.extras["w_k"][h]
        want = (mq @ mk.T) / math.sqrt(D)
        # proj_q holds W_q W_k^T - I rounded to fp32: agreement to fp32 rounding
        np.testing.assert_allclose(s[h], want, rtol=1e-5, atol=1e-6)
        # and the rankings per row agree (what selection uses)
        assert (np.argsort(-s[h], axis=1, kind="stable")[:, :2] ==
                np.argsort(-want, axis=1, kind="stable")[:, :2]).all()


def test_logits_linear_projection_example():
    # one head, D=2, one tile each: f = [m | mx | mn] (6 values), P picked by hand
    fq = np.array([[[1.0, 2.0, 3.0, 4.0, 5.0, 6.0]]])
    fk = np.array([[[0.5, -1.0, 0.0, 1.0, 2.0, 0.0]]])
    P = np.zeros((1, 6, 2))
    P[0, 2, 0] = 1.0     # q_hat_0 = m0 + mx0 = 1 + 3 = 4
    P[0, 5, 1] = -1.0    # q_hat_1 = m1 - mn1 = 2 - 6 = -4
    Pk = np.zeros((1, 6, 2))
    Pk[0, 4, 1] = 0.5    # k_hat = (0.5, -1 + 0.5*2) = (0.5, 0)
    s = predictor.logits(fq, fk, P, Pk)
    assert s[0, 0, 0] == pytest.approx((4 * 0.5 + (-4) * 0.0) / math.sqrt(2), abs=1e-15)
