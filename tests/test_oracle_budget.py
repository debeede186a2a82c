"""Pins for the oracle's budget algebra (veda_core.py, section "budgets")."""
import math
import os
import random
from fractions import Fraction

import numpy as np
import pytest

from conftest import GOLDEN
from oracle import budget, tiles
import workloads


def _golden_bresenham():
    out = []
    for line in open(os.path.join(GOLDEN, "bresenham.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        left, right = line.split("->")
        n, f = left.split()
        out.append((int(n), float(f), [int(x) for x in right.split()]))
    return out


def _golden_splits():
    out = []
    for line in open(os.path.join(GOLDEN, "budget_splits.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        left, right = line.split("->")
        name, block, n, nv = left.split()
        lo, hi, frac, extra = right.split()
        out.append((name, block, int(n), int(nv), int(lo), int(hi), float(frac), int(extra)))
    return out


def test_sparsity_is_one_minus_share():
    assert budget.sparsity_budget(0.9) == (0.09999999999999998, None)
    assert budget.sparsity_budget(0.9)[0] != 0.1
    assert budget.keeps_all((1.0, None)) and budget.keeps_all((1.5, None))
    assert not budget.keeps_all((0.99, None)) and not budget.keeps_all((None, 1e9))


@pytest.mark.parametrize("n,f,rows", _golden_bresenham())
def test_bresenham_hand_examples(n, f, rows):
    e = budget.bresenham(n, f)
    assert np.nonzero(e)[0].tolist() == rows


@pytest.mark.parametrize("seed", range(5))
def test_bresenham_total_is_floor_n_f(seed):
    rng = random.Random(seed)
    for _ in range(200):
        n = rng.randint(1, 3000)
        f = round(rng.random(), 12)
        e = budget.bresenham(n, f)
        # the pattern telescopes: sum_r [F(r+1) > F(r)] = F(n) with F(r) = floor(r f)
        assert int(e.sum()) == math.floor(n * f)
        # prefix property used to size rows without a scan: sum_{r'<r} e = floor(r f)
        r = rng.randint(0, n)
        assert int(e[:r].sum()) == math.floor(r * f)


def _block_of(name, block):
    wl = workloads.get(name.split("_")[0])
    gen = budget.from_request(wl.generated)
    ref = budget.from_request(wl.reference)
    if block == "ref":
        start, g = wl.refs[0]
        return ref, g[0] * g[1] * g[2]
    g = wl.target[1]
    return gen, g[0] * g[1] * g[2]


@pytest.mark.parametrize("row", _golden_splits(), ids=lambda r: f"{r[0]}-{r[1]}")
def test_split_per_workload_hand_values(row):
    name, block, n, nv, lo, hi, frac, extra = row
    bud, real = _block_of(name, block)
    got = budget.split(budget.per_row(bud, real, n), n)
    assert got == (lo, hi, frac)
    assert int(budget.bresenham(nv, got[2]).sum()) == extra


def test_split_bounds_and_rounding():
    rng = random.Random(7)
    for _ in range(20000):
        n = rng.randint(1, 2500)
        b = rng.uniform(0, 1.2 * n)
        lo, hi, frac = budget.split(b, n)
        assert 1 <= lo <= hi <= n
        if b >= n:
            assert (lo, hi, frac) == (n, n, 0.0)
            continue
        assert hi == min(lo + 1, n)
        assert 0.0 <= frac <= 1.0
        want = min(max(b - lo, 0.0), 1.0)
        # frac is the 12-decimal rounding of b - lo: check against exact rationals
        exact = Fraction(want)
        assert abs(Fraction(frac) - exact) <= Fraction(1, 2 * 10 ** 12) + Fraction(1, 10 ** 16)
        if b >= 1:
            assert lo == math.floor(b)


def test_per_row_equal_cost_rule():
    # a ratio budget is priced on the unpadded tile count: padding columns never
    # raise the per-row budget above ratio * ideal
    for real, n in [(1200, 18), (104160, 837), (4032, 33), (219600, 1830), (219600, 1920)]:
        ideal = -(-real // 128)
        b = budget.per_row((0.1, None), real, n)
        assert b * n == pytest.approx(0.1 * ideal * ideal, rel=1e-15)
        assert b <= 0.1 * ideal + 1e-9
    assert budget.per_row((None, 24.0), 10 ** 6, 5) == 24.0
