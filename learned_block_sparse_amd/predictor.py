"""The predictor file and its tile plans (page `veda_core.py`, section "tile
plans and the predictor file").

A predictor file is a safetensors file whose metadata names the format, the
model's layer and head counts, the budgets it was trained with and its tile
plans (JSON), and whose tensors are the per-layer projections proj_q and
proj_k of shape [heads, 3 * head_dim, head_dim], stored as float32, bfloat16
or float8_e4m3fn (the last with a per-head scale tensor beside each). It is
read strictly: every declared tensor must be present with its shape, and
nothing else may be.

A tile plan is a latent grid the predictor was trained on, a list of tile
boxes, and per layer and head the index of the box that head uses. For a
video of another size the plan with the nearest aspect ratio, then the
nearest length, then the least padding is taken, the H <-> W mirror of
every plan competing too; the result says whether it is an exact match.

Host-side reading and choosing only: the projections go to the device when a
layer is attended (`layer_inputs`), and every step of attention runs in
libveda's kernels.
"""
from __future__ import annotations

import json
import math
import os
from dataclasses import dataclass, field

FORMAT = "miowtion-veda-predictor-v1"
FPS = 24                     # frames per second of the model's videos
_DTYPES = ("float32", "bfloat16", "float8_e4m3fn")


class PredictorError(ValueError):
    """A predictor file that cannot be used; the text says why."""


@dataclass
class TilePlan:
    """One trained tile plan: grid (T, H, W), the boxes, and per layer the
    index into `shapes` of each head's box."""
    name: str
    grid: tuple
    shapes: list
    head_shape: list
    _groups: dict = field(default_factory=dict, repr=False)

    def mirrored(self) -> "TilePlan":
        """The same plan for the transposed frame: H and W swap in the grid
        and in every box."""
        T, H, W = self.grid
        return TilePlan(self.name + "_T", (T, W, H), [(t, w, h) for t, h, w in self.shapes],
                        self.head_shape)

    def head_groups(self, layer: int):
        """[(box, [heads])] of one layer: the heads that share a box, in the
        order of the boxes' indices."""
        if layer not in self._groups:
            row = self.head_shape[layer]
            self._groups[layer] = [(self.shapes[i], [h for h, j in enumerate(row) if j == i])
                                   for i in sorted(set(row))]
        return self._groups[layer]

    def layer_head_shapes(self, layer: int):
        """Per head, its box for `layer` (the `head_shapes` argument of
        attention())."""
        return [self.shapes[i] for i in self.head_shape[layer]]


@dataclass
class Predictor:
    """A read predictor file."""
    path: str
    layers: int
    heads: int
    dim: int
    generated: tuple          # budget request, ('ratio', r) or ('tiles', n)
    reference: tuple
    plans: list
    proj_q: list              # per layer, torch bfloat16 [heads, 3 dim, dim] on the host
    proj_k: list
    meta: dict


def _tiles_for(grid, box):
    n = 1
    for g, s in zip(grid, box):
        n *= -(-g // s)
    return n


def describe_grid(grid) -> str:
    """'<width>x<height>, <seconds> s' of a latent grid (T, H, W): 32 pixels
    per latent cell, and 17 n + 5 frames for a latent length of 5 n + 2 (one
    frame below two), at FPS frames per second."""
    T, H, W = (int(x) for x in grid)
    frames = 17 * ((T - 2) // 5) + 5 if T >= 2 else 1
    return f"{W * 32}x{H * 32}, {frames / FPS:.1f} s"


def describe_budget(request) -> str:
    kind, value = request
    if kind == "tiles":
        return f"{value:g} tiles"
    ratio = 1.0 - value if kind == "sparsity" else value
    return f"{100.0 * (1.0 - min(ratio, 1.0)):g}% sparse"


def describe_predictor(p: Predictor) -> str:
    trained = describe_budget(p.generated)
    if p.reference != p.generated:
        trained += f" / reference {describe_budget(p.reference)}"
    return f"{os.path.basename(p.path)}, {p.layers} layers x {p.heads} heads, trained {trained}"


def choose_plan(plans, grid):
    """(plan, exact, words) for a video of latent grid (T, H, W).

    Every plan and its H <-> W mirror compete. The winner has, in order of
    priority: the log aspect ratio (W / H) nearest the video's (distances
    compared at 3 decimals), the nearest latent length T, the fewest tiles
    over all of the plan's boxes on this grid; the first candidate wins a
    full tie (the plans in file order, then their mirrors). A plan of another
    size still tiles any grid, so this never fails; `exact` is whether the
    plan was trained for this very grid, and `words` says which size it was
    trained for.
    """
    grid = tuple(int(g) for g in grid)
    if not plans:
        raise PredictorError("no tile plans to choose from")
    want = math.log(grid[2] / grid[1])

    def key(p):
        return (round(abs(math.log(p.grid[2] / p.grid[1]) - want), 3),
                abs(p.grid[0] - grid[0]),
                sum(_tiles_for(grid, s) for s in p.shapes))

    best = None
    for p in list(plans) + [p.mirrored() for p in plans]:
        if best is None or key(p) < key(best):
            best = p
    if best.grid == grid:
        return best, True, f"trained for this size ({describe_grid(grid)})"
    return best, False, (f"nearest trained size: {describe_grid(best.grid)} "
                         f"(this video: {describe_grid(grid)})")


def read_metadata(path) -> dict:
    from safetensors import safe_open
    name = os.path.basename(path)
    try:
        with safe_open(path, framework="pt", device="cpu") as f:
            meta = dict(f.metadata() or {})
    except Exception as exc:  # noqa: BLE001 - the reader raises several types
        raise PredictorError(f"{name}: cannot be read as safetensors ({exc})") from exc
    if meta.get("format") != FORMAT:
        raise PredictorError(f"{name}: format is {meta.get('format')!r}, a Veda predictor "
                             f"file declares {FORMAT!r}")
    return meta


def _budget(meta, prefix, default, name):
    kind = meta.get(f"{prefix}_budget_kind")
    if kind is None:
        return default
    if kind not in ("ratio", "tiles"):
        raise PredictorError(f"{name}: {prefix}_budget_kind must be 'ratio' or 'tiles', "
                             f"not {kind!r}")
    try:
        value = float(meta[f"{prefix}_budget_value"])
    except (KeyError, ValueError) as exc:
        raise PredictorError(f"{name}: {prefix}_budget_value is missing or not a number "
                             f"({exc})") from exc
    return (kind, value)


def _box(text, name):
    try:
        box = tuple(int(x) for x in text.split("x"))
    except ValueError:
        box = ()
    if len(box) != 3 or any(b <= 0 or b & (b - 1) for b in box) or box[0] * box[1] * box[2] != 128:
        raise PredictorError(f"{name}: tile box {text!r} is not t x h x w powers of two with "
                             "128 cells")
    return box


def load_predictor(path) -> Predictor:
    """Reads a predictor file strictly (see the module text). Projections
    stay on the host in bfloat16; float8 ones are scaled per head on the way
    (value times that head's scale), then rounded to bfloat16."""
    import torch
    from safetensors import safe_open
    meta = read_metadata(path)
    name = os.path.basename(path)
    try:
        layers, heads, dim = (int(meta[k]) for k in ("num_layers", "num_heads", "head_dim"))
        keep = meta.get("keep_ratio")
        generated = _budget(meta, "target", None if keep is None else ("ratio", float(keep)),
                            name)
        if generated is None:
            raise KeyError("target_budget_kind (or keep_ratio)")
        reference = _budget(meta, "ref", generated, name)
        plans_json = json.loads(meta["plans"])
    except (KeyError, ValueError) as exc:
        raise PredictorError(f"{name}: metadata incomplete ({exc})") from exc
    if min(layers, heads, dim) <= 0:
        raise PredictorError(f"{name}: layer, head and head_dim counts must be positive")
    stored = meta.get("dtype", "float32")
    if stored not in _DTYPES:
        raise PredictorError(f"{name}: tensors stored as {stored!r}, not one of {_DTYPES}")
    with safe_open(path, framework="pt", device="cpu") as f:
        tensors = {k: f.get_tensor(k) for k in f.keys()}
    want = (heads, 3 * dim, dim)
    proj = {"proj_q": [], "proj_k": []}
    for layer in range(layers):
        for kind, out in proj.items():
            key = f"layers.{layer}.{kind}"
            value = tensors.pop(key, None)
            if value is None or tuple(value.shape) != want:
                got = "absent" if value is None else list(value.shape)
                raise PredictorError(f"{name}: {key} must be {list(want)}, found {got}")
            if stored == "float8_e4m3fn":
                scale = tensors.pop(key + ".__scale", None)
                if scale is None or tuple(scale.shape) != (heads,):
                    raise PredictorError(f"{name}: {key} is float8 without a [{heads}] "
                                         "per-head scale")
                value = value.float() * scale.float().view(-1, 1, 1)
            out.append(value.to(torch.bfloat16).contiguous())
    if tensors:
        raise PredictorError(f"{name}: tensors the metadata does not declare: "
                             f"{sorted(tensors)[:4]}")
    plans = []
    for entry in (plans_json.values() if isinstance(plans_json, dict) else plans_json):
        try:
            plan = TilePlan(str(entry["geometry"]), tuple(int(x) for x in entry["grid"]),
                            [_box(s, name) for s in entry["shapes"]],
                            [[int(i) for i in row] for row in entry["head_shape"]])
        except (KeyError, TypeError, ValueError) as exc:
            raise PredictorError(f"{name}: a tile plan is malformed ({exc})") from exc
        if len(plan.grid) != 3 or min(plan.grid) <= 0:
            raise PredictorError(f"{name}: plan {plan.name} has grid {plan.grid}")
        if len(plan.head_shape) != layers or any(len(r) != heads for r in plan.head_shape):
            raise PredictorError(f"{name}: plan {plan.name} does not give a box to each of "
                                 f"{layers} layers x {heads} heads")
        if any(not 0 <= i < len(plan.shapes) for r in plan.head_shape for i in r):
            raise PredictorError(f"{name}: plan {plan.name} names a box it does not list")
        plans.append(plan)
    if not plans:
        raise PredictorError(f"{name}: the file holds no tile plan")
    return Predictor(path, layers, heads, dim, generated, reference, plans, proj["proj_q"],
                     proj["proj_k"], meta)


def layer_inputs(pred: Predictor, plan: TilePlan, layer: int, device):
    """(head_shapes, proj_q, proj_k) for attention() on one layer: each
    head's box from the plan, and the layer's projections on `device` as
    float32 [heads, 3 dim, dim]."""
    if not 0 <= layer < pred.layers:
        raise PredictorError(f"layer {layer} not in [0, {pred.layers})")
    return (plan.layer_head_shapes(layer),
            pred.proj_q[layer].to(device).float().contiguous(),
            pred.proj_k[layer].to(device).float().contiguous())
