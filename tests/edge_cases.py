"""Small hand-made layer geometries that the five benchmark workloads do not
cover (inputs only, no method arithmetic): shared by the oracle pins and the
GPU parity tests."""
import dataclasses

import workloads

_base = workloads.get("padding")

EDGE = {
    # one video cell (a tile with a single real row) between text rows
    "one_cell": dataclasses.replace(
        _base, name="one_cell", index=11, seq_len=10, n_heads=2,
        target=(3, (1, 1, 1)), head_shapes=(None, None), generated=("ratio", 0.5),
        reference=("ratio", 0.5)),
    # two reference spans and a ragged target, globals before, between and after
    "ragged_refs": dataclasses.replace(
        _base, name="ragged_refs", index=12, seq_len=700, n_heads=3,
        head_dim=128, refs=((5, (1, 5, 6)), (40, (2, 3, 4))), target=(90, (3, 5, 37)),
        head_shapes=(None, (1, 8, 16), None), generated=("sparsity", 0.5),
        reference=("sparsity", 0.6)),
    # keep-all budget: must equal dense attention
    "keep_all": dataclasses.replace(_base, name="keep_all", index=13,
                                    generated=("ratio", 1.0), reference=("ratio", 1.0)),
    # a tile budget larger than the block
    "tiles_big": dataclasses.replace(_base, name="tiles_big", index=14,
                                     generated=("tiles", 100.0), reference=("tiles", 100.0)),
    # fp32 with global rows and padding
    "f32_padding": dataclasses.replace(_base, name="f32_padding", index=15,
                                       dtype="f32", head_dim=128),
    # head_dim 64 over many tiles: locality bias, a reference span, a ragged
    # target (w = 46), text rows before and after, and five heads in three
    # tile boxes (a group of three heads, and two single-head groups)
    "d64_bias": dataclasses.replace(
        _base, name="d64_bias", index=17, seq_len=11000, n_heads=5, head_dim=64,
        refs=((64, (1, 24, 40)),), target=(1024, (9, 24, 46)),
        head_shapes=(None, (1, 8, 16), None, (2, 8, 8), (4, 4, 8)),
        generated=("sparsity", 0.8), reference=("sparsity", 0.7), bias=True),
    # the most heads one call takes (VEDA_MAX_HEADS)
    "max_heads": dataclasses.replace(_base, name="max_heads", index=18, n_heads=256,
                                     head_shapes=(None,) * 256),
    # the most spans one plan takes (VEDA_MAX_SPANS): 15 one-tile references,
    # each with text rows before it, then the target
    "max_spans": dataclasses.replace(
        _base, name="max_spans", index=19, seq_len=15 * 40 + 8 + 512 + 24, n_heads=2,
        refs=tuple((8 + 40 * i, (1, 4, 8)) for i in range(15)), target=(608, (2, 16, 16)),
        head_shapes=(None, None), generated=("ratio", 0.3), reference=("ratio", 0.4)),
    # a reference span whose budget keeps everything: it is not tiled, its
    # rows join the text rows as global rows
    "refs_whole": dataclasses.replace(
        _base, name="refs_whole", index=16, seq_len=1500, n_heads=4,
        refs=((0, (2, 5, 12)),), target=(130, (5, 12, 20)), head_shapes=(None,) * 4,
        generated=("ratio", 0.25), reference=("ratio", 1.0)),
}


def get(name):
    return EDGE.get(name) or workloads.get(name)
