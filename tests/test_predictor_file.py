"""The predictor file reader and tile-plan choice (veda_core.py, page 1,
section "tile plans and the predictor file") on synthetic files: the real
predictor is not available, so files of the same format are written here.
Pinned against hand-derived choices (tests/golden/plan_choice.txt), the
oracle's independent choice rule over random grids, the page's receipt line
("1344x768 · 5.2 s" for 124 frames) and an independent float8 decoder."""
import json
import os
import random

import numpy as np
import pytest
import torch
from safetensors.torch import save_file

from conftest import GOLDEN
from learned_block_sparse_amd import predictor as P
from oracle import plans as OP

PLANS = {
    "a": {"geometry": "wide_5s", "grid": [37, 24, 42], "shapes": ["1x8x16", "8x4x4"],
          "head_shape": [[0, 1, 0], [1, 1, 0]]},
    "b": {"geometry": "wide_10s", "grid": [72, 24, 42], "shapes": ["1x8x16", "8x4x4"],
          "head_shape": [[0, 0, 0], [1, 1, 1]]},
    "c": {"geometry": "square", "grid": [37, 24, 24], "shapes": ["2x8x8"],
          "head_shape": [[0, 0, 0], [0, 0, 0]]},
    "d": {"geometry": "wide_b", "grid": [37, 24, 42], "shapes": ["4x4x8"],
          "head_shape": [[0, 0, 0], [0, 0, 0]]},
}
L, H, D = 2, 3, 16


def _meta(**over):
    m = {"format": P.FORMAT, "num_layers": str(L), "num_heads": str(H), "head_dim": str(D),
         "target_budget_kind": "ratio", "target_budget_value": "0.1", "plans": json.dumps(PLANS)}
    m.update({k: v for k, v in over.items() if v is not None})
    for k in [k for k, v in over.items() if v is None]:
        m.pop(k, None)
    return m


def _tensors(dtype="float32", seed=0):
    g = torch.Generator().manual_seed(seed)
    t = {}
    for layer in range(L):
        for kind in ("proj_q", "proj_k"):
            x = torch.randn(H, 3 * D, D, generator=g) * 0.3
            key = f"layers.{layer}.{kind}"
            if dtype == "float8_e4m3fn":
                t[key] = x.to(torch.float8_e4m3fn)
                t[key + ".__scale"] = torch.rand(H, generator=g) + 0.5
            else:
                t[key] = x.to(getattr(torch, dtype))
    return t


def _write(tmp_path, tensors, meta, name="pred.safetensors"):
    path = os.path.join(tmp_path, name)
    save_file(tensors, path, metadata=meta)
    return path


@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "float8_e4m3fn"])
def test_reads_projections_in_every_storage_dtype(tmp_path, dtype):
    t = _tensors(dtype)
    pred = P.load_predictor(_write(tmp_path, t, _meta(dtype=dtype)))
    assert (pred.layers, pred.heads, pred.dim) == (L, H, D)
    for layer in range(L):
        for kind, got in (("proj_q", pred.proj_q[layer]), ("proj_k", pred.proj_k[layer])):
            key = f"layers.{layer}.{kind}"
            assert got.dtype == torch.bfloat16 and tuple(got.shape) == (H, 3 * D, D)
            if dtype == "float8_e4m3fn":
                codes = t[key].view(torch.uint8).numpy()
                want = OP.dequantize(codes, t[key + ".__scale"].numpy())
            else:
                want = OP.to_bf16(t[key].float().numpy())
            assert np.array_equal(got.float().numpy(), want), key


def test_budgets_from_metadata(tmp_path):
    t = _tensors()
    p = P.load_predictor(_write(tmp_path, t, _meta()))
    assert p.generated == ("ratio", 0.1) and p.reference == ("ratio", 0.1)
    p = P.load_predictor(_write(tmp_path, t, _meta(target_budget_kind=None,
                                                   target_budget_value=None, keep_ratio="0.05")))
    assert p.generated == ("ratio", 0.05)
    p = P.load_predictor(_write(tmp_path, t, _meta(ref_budget_kind="tiles",
                                                   ref_budget_value="24")))
    assert p.reference == ("tiles", 24.0)
    assert "10 tiles" not in P.describe_predictor(p) and "90% sparse" in P.describe_predictor(p)
    assert "24 tiles" in P.describe_predictor(p)


@pytest.mark.parametrize("case,match", [
    ("format", "format is"),
    ("missing", "must be"),
    ("shape", "must be"),
    ("extra", "does not declare"),
    ("fp8_noscale", "per-head scale"),
    ("kind", "must be 'ratio' or 'tiles'"),
    ("value", "budget_value"),
    ("nobudget", "metadata incomplete"),
    ("noplans", "no tile plan"),
    ("plan_dims", "does not give a box"),
    ("plan_box", "tile box"),
    ("plan_index", "does not list"),
    ("dtype", "stored as"),
    ("garbage", "cannot be read"),
])
def test_refuses_malformed_files(tmp_path, case, match):
    t, m = _tensors(), _meta()
    if case == "format":
        m["format"] = "something-else"
    elif case == "missing":
        del t["layers.1.proj_k"]
    elif case == "shape":
        t["layers.0.proj_q"] = t["layers.0.proj_q"][:, :D].contiguous()
    elif case == "extra":
        t["layers.2.proj_q"] = t["layers.0.proj_q"].clone()
    elif case == "fp8_noscale":
        t = _tensors("float8_e4m3fn")
        del t["layers.0.proj_q.__scale"]
        m["dtype"] = "float8_e4m3fn"
    elif case == "kind":
        m["target_budget_kind"] = "percent"
    elif case == "value":
        m["target_budget_value"] = "ten"
    elif case == "nobudget":
        del m["target_budget_kind"]
    elif case == "noplans":
        m["plans"] = "{}"
    elif case == "plan_dims":
        bad = dict(PLANS)
        bad["a"] = dict(PLANS["a"], head_shape=[[0, 1, 0]])
        m["plans"] = json.dumps(bad)
    elif case == "plan_box":
        m["plans"] = json.dumps({"a": dict(PLANS["a"], shapes=["1x8x8", "8x4x4"])})
    elif case == "plan_index":
        m["plans"] = json.dumps({"a": dict(PLANS["a"], head_shape=[[0, 2, 0], [1, 1, 0]])})
    elif case == "dtype":
        m["dtype"] = "int8"
    if case == "garbage":
        path = os.path.join(tmp_path, "junk.safetensors")
        open(path, "wb").write(b"not a safetensors file at all")
    else:
        path = _write(tmp_path, t, m)
    with pytest.raises(P.PredictorError, match=match):
        P.load_predictor(path)


def _golden_choices():
    out = []
    for line in open(os.path.join(GOLDEN, "plan_choice.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        left, right = line.split("->")
        name, exact = right.split()
        out.append((tuple(int(x) for x in left.split()), name, exact == "1"))
    return out


@pytest.mark.parametrize("grid,name,exact", _golden_choices())
def test_plan_choice_matches_hand_derivation(tmp_path, grid, name, exact):
    pred = P.load_predictor(_write(tmp_path, _tensors(), _meta()))
    plan, is_exact, words = P.choose_plan(pred.plans, grid)
    assert (plan.name, is_exact) == (name, exact)
    assert words.startswith("trained for this size" if exact else "nearest trained size")


def _oracle_plans():
    return [(p["geometry"], tuple(p["grid"]), [tuple(int(x) for x in s.split("x"))
                                                for s in p["shapes"]], p["head_shape"])
            for p in PLANS.values()]


def test_plan_choice_matches_oracle_on_random_grids(tmp_path):
    pred = P.load_predictor(_write(tmp_path, _tensors(), _meta()))
    rng = random.Random(7)
    for _ in range(2000):
        grid = (rng.randint(1, 90), rng.randint(1, 60), rng.randint(1, 60))
        plan, exact, _ = P.choose_plan(pred.plans, grid)
        name, g, oexact = OP.choose_plan(_oracle_plans(), grid)
        assert (plan.name, plan.grid, exact) == (name, g, oexact), grid


def test_head_groups_and_layer_shapes(tmp_path):
    pred = P.load_predictor(_write(tmp_path, _tensors(), _meta()))
    for plan in pred.plans + [p.mirrored() for p in pred.plans]:
        for layer in range(L):
            want = OP.head_groups(plan.shapes, plan.head_shape[layer])
            assert plan.head_groups(layer) == want
            shapes = plan.layer_head_shapes(layer)
            assert [shapes[h] for _, hs in want for h in hs] == \
                [s for s, hs in want for _ in hs]
    wide = pred.plans[0]
    assert wide.head_groups(0) == [((1, 8, 16), [0, 2]), ((8, 4, 4), [1])]
    assert wide.mirrored().head_groups(0) == [((1, 16, 8), [0, 2]), ((8, 4, 4), [1])]


@pytest.mark.parametrize("grid,text", [
    ((37, 24, 42), "1344x768, 5.2 s"),      # 124 frames: the node's receipt for its demo
    ((72, 24, 42), "1344x768, 10.1 s"),      # 243 frames
    ((1, 24, 24), "768x768, 0.0 s"),
])
def test_describe_grid(grid, text):
    assert P.describe_grid(grid) == text == OP.describe_grid(grid)


def test_layer_inputs_on_cpu(tmp_path):
    pred = P.load_predictor(_write(tmp_path, _tensors("bfloat16"), _meta(dtype="bfloat16")))
    plan = pred.plans[0]                               # wide_5s
    shapes, pq, pk = P.layer_inputs(pred, plan, 1, "cpu")
    assert shapes == [(8, 4, 4), (8, 4, 4), (1, 8, 16)]
    assert pq.dtype == torch.float32 and tuple(pq.shape) == (H, 3 * D, D)
    assert torch.equal(pq, pred.proj_q[1].float())
    with pytest.raises(P.PredictorError):
        P.layer_inputs(pred, plan, L, "cpu")
