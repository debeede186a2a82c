"""Pins for the oracle's teacher map and recall (oracle/teacher.py): a
pure-Python brute force of the definition on tiny layouts, closed forms
(equal scores; one dominant key) and invariants."""
import itertools
import math

import numpy as np
import pytest

from oracle import teacher, tiles


def _layout(T, H, W, box, text=0):
    return tiles.build_layout([(0, (T, H, W), box)], T * H * W + text)


def _brute(q, k, lay, h, a, b):
    """max over real i in a, real j in b of softmax_j(q_i . k_j / sqrt D),
    with plain loops over every real key."""
    D = q.shape[2]
    real = [r for t in range(lay.n_tiles) for r in lay.tile_rows(t)]
    best = 0.0
    for i in lay.tile_rows(a):
        logits = [sum(float(q[i, h, d]) * float(k[j, h, d]) for d in range(D)) / math.sqrt(D)
                  for j in real]
        m = max(logits)
        z = sum(math.exp(x - m) for x in logits)
        for j in lay.tile_rows(b):
            p = math.exp(logits[real.index(j)] - m) / z
            best = max(best, p)
    return best


def test_matches_brute_force_on_a_padded_layout_with_text():
    rng = np.random.default_rng(1)
    lay = _layout(1, 5, 30, (1, 8, 16), text=20)      # 2 video tiles (80 + 70 rows) + 1 text tile
    S = lay.seq_len
    q = rng.standard_normal((S, 2, 4))
    k = rng.standard_normal((S, 2, 4))
    T = teacher.teacher_map(q, k, lay, [0, 1])
    for h, a, b in itertools.product(range(2), range(lay.n_tiles), range(lay.n_tiles)):
        assert abs(T[h, a, b] - _brute(q, k, lay, h, a, b)) <= 1e-12


def test_equal_scores_give_uniform_teacher():
    lay = _layout(2, 8, 16, (1, 8, 16), text=50)      # 2 video tiles + 1 text tile
    S = lay.seq_len
    q = np.zeros((S, 1, 8))
    k = np.random.default_rng(2).standard_normal((S, 1, 8))
    T = teacher.teacher_map(q, k, lay, [0])
    assert np.allclose(T, 1.0 / S, rtol=0, atol=1e-15)
    mask = np.zeros((1, lay.n_tiles, lay.n_tiles), dtype=bool)
    mask[0, :, 0] = True
    assert np.allclose(teacher.recall(T, mask), 1.0 / lay.n_tiles)


def test_dominant_key_takes_the_teacher_mass():
    lay = _layout(1, 8, 64, (1, 8, 16))                # 4 tiles of 128
    S, D = lay.seq_len, 8
    rng = np.random.default_rng(3)
    q = rng.standard_normal((S, 1, D)) * 0.01
    k = rng.standard_normal((S, 1, D)) * 0.01
    j = lay.tile_rows(2)[17]
    q[:, 0, :] += 1.0
    k[j, 0, :] = 40.0                                   # every query's scores peak at row j
    T = teacher.teacher_map(q, k, lay, [0])
    dist = teacher.teacher_distribution(T)
    assert (dist[0, :, 2] > 1 - 1e-12).all()
    keep2 = np.zeros((1, 4, 4), dtype=bool)
    keep2[0, :, 2] = True
    assert np.allclose(teacher.recall(T, keep2), 1.0)
    assert (teacher.recall(T, ~keep2) < 1e-12).all()


def test_invariants_and_query_tile_sampling():
    rng = np.random.default_rng(4)
    lay = _layout(3, 8, 16, (1, 8, 16), text=40)
    S = lay.seq_len
    q = rng.standard_normal((S, 2, 16))
    k = rng.standard_normal((S, 2, 16))
    T = teacher.teacher_map(q, k, lay, [0, 1])
    assert ((T > 0) & (T <= 1)).all()
    # every query row's probabilities sum to 1, so its largest is >= 1/S and
    # the tile maxima over one query tile add to at least that
    assert (T.max(axis=-1) >= 1.0 / S).all()
    # a sample of query tiles gives the same rows
    Ts = teacher.teacher_map(q, k, lay, [0, 1], query_tiles=[3, 1])
    assert np.array_equal(Ts[:, 0], T[:, 3]) and np.array_equal(Ts[:, 1], T[:, 1])
    # the keep-all mask recalls everything
    full = np.ones((2, lay.n_tiles, lay.n_tiles), dtype=bool)
    assert np.allclose(teacher.recall(T, full), 1.0)
