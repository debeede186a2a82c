"""libveda on the CPU: the library loads, exports every entry point its header
declares, and its host-side logic (span validation, least-padding boxes,
layout sizes, budget splits with Python's rounding, CSR sizing) agrees with
the oracle. No kernel is launched here."""
import math
import os
import random
import re
import subprocess
import sys

import numpy as np
import pytest

import learned_block_sparse_amd as veda
from learned_block_sparse_amd import _lib
from oracle import tiles, budget, selection, layer
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


HOST_ONLY_EXPORTS = {"veda_last_error", "veda_version", "veda_plan_query", "veda_select_query",
                     "veda_attend_check", "veda_attend_int8_query"}


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    header = open(os.path.join(ROOT, "include", "veda.h")).read()
    declared = set(re.findall(r"\b(veda_[a-z_0-9]+)\s*\(", header))
    assert declared == set(_lib.EXPORTS)
    # a host-only build (the sanitizer run) carries just the host entry points
    for name in (declared if _lib.has_kernels() else HOST_ONLY_EXPORTS):
        assert hasattr(lib, name), name
    assert "gfx950" in veda.version()


def _spans(wl, shape, tile_refs=True):
    sp = [(s, g, None) for s, g in wl.refs] if tile_refs else []
    sp.append((wl.target[0], wl.target[1], shape))
    return sp


@pytest.mark.parametrize("name", ["tiny", "padding", "mid", "headline", "long"])
def test_plan_query_matches_oracle_layout(name):
    wl = workloads.get(name)
    for shape in sorted(set(wl.head_shapes), key=str):
        info = veda.veda_plan_query(_spans(wl, shape), wl.seq_len)
        oshape = tiles.least_padding_shape(wl.target[1]) if shape is None else shape
        ospans = [(s, g, tiles.least_padding_shape(g)) for s, g in wl.refs]
        ospans.append((wl.target[0], wl.target[1], oshape))
        lay = tiles.build_layout(ospans, wl.seq_len)
        assert (info.n_tiles, info.n_video, info.n_ref, info.n_global) == \
            (lay.n_tiles, lay.n_video, lay.n_ref, lay.n_global)
        assert info.n_slots == lay.n_slots
        assert (info.ref_tokens, info.target_tokens) == (lay.ref_tokens, lay.target_tokens)
        for i, (_, _, s) in enumerate(ospans):
            assert tuple(info.spans[i].shape) == tuple(s)


@pytest.mark.parametrize("grid", [(5, 12, 20), (31, 48, 70), (1, 48, 84), (61, 45, 80),
                                  (1, 1, 1), (3, 200, 7), (130, 1, 1), (2, 2, 2)])
def test_least_padding_choice_matches_oracle(grid):
    info = veda.veda_plan_query([(0, grid, None)], grid[0] * grid[1] * grid[2])
    assert tuple(info.spans[0].shape) == tiles.least_padding_shape(grid)


@pytest.mark.parametrize("spans,seq", [
    ([], 10),
    ([(0, (1, 8, 8), (1, 8, 16)), (32, (1, 8, 8), (1, 8, 16))], 200),
    ([(0, (1, 8, 8), (1, 8, 16))], 63),
    ([(-1, (1, 8, 8), (1, 8, 16))], 100),
    ([(0, (1, 8, 8), (1, 8, 8))], 100),          # not a 128-cell box
    ([(0, (0, 8, 8), None)], 100),               # empty grid
])
def test_plan_query_refuses_like_the_oracle(spans, seq):
    with pytest.raises(veda.VedaError):
        veda.veda_plan_query(spans, seq)
    ospans = [(s, g, sh if sh is not None else (1, 8, 16)) for s, g, sh in spans]
    if all(sh is None or sh[0] * sh[1] * sh[2] == 128 for _, _, sh in spans) and \
            all(min(g) > 0 for _, g, _ in spans):
        with pytest.raises(tiles.VedaError):
            tiles.build_layout(ospans, seq)


@pytest.mark.parametrize("name", ["tiny", "padding", "mid", "headline", "long"])
def test_select_query_matches_oracle_blocks_and_sizes(name):
    wl = workloads.get(name)
    gen, ref = budget.from_request(wl.generated), budget.from_request(wl.reference)
    for shape in sorted(set(wl.head_shapes), key=str):
        info = veda.veda_plan_query(_spans(wl, shape), wl.seq_len)
        sel = veda.veda_select_query(info, veda.budget(wl.generated), veda.budget(wl.reference),
                                     wl.head_dim, wl.n_heads)
        oshape = tiles.least_padding_shape(wl.target[1]) if shape is None else shape
        lay = layer.layout_for(wl, oshape, gen, ref)
        blocks = selection.column_blocks(lay, gen, ref)
        params = selection.block_params(lay, blocks)
        assert sel.n_blocks == len(params)
        for b, (start, stop, keep_all, lo, hi, frac) in enumerate(params):
            k = sel.blocks[b]
            assert (k.start, k.stop, bool(k.keep_all), k.k_lo, k.k_hi) == (start, stop, keep_all, lo, hi)
            assert k.frac == frac                      # bit-identical double
        # CSR size: closed form per row, summed
        nv = lay.n_video
        want = sum(nv * lo + math.floor(nv * frac) for (_, _, _, lo, _, frac) in params)
        want += nv * lay.n_global + lay.n_global * lay.n_tiles
        assert sel.entries_per_head == want


@pytest.mark.parametrize("name", ["tiny", "padding", "mid"])
def test_select_query_entries_equal_oracle_mask(name):
    inp = workloads.generate(name)
    wl = inp.workload
    groups, _ = layer.run(inp, do_attend=False)
    for g in groups:
        info = veda.veda_plan_query(_spans(wl, g.shape), wl.seq_len)
        sel = veda.veda_select_query(info, veda.budget(wl.generated), veda.budget(wl.reference),
                                     wl.head_dim, len(g.heads))
        per_head = g.mask.sum(axis=(1, 2))
        assert (per_head == sel.entries_per_head).all()
        assert sel.widest == g.mask.sum(axis=2).max()


def test_budget_split_matches_python_rounding():
    """Tile budgets b over n columns give frac = round(b - floor(b), 12):
    libveda's decimal rounding (printf + strtod) against Python's round()."""
    rng = random.Random(1234)
    info = veda.veda_plan_query([(0, (1, 8, 16 * 4000), (1, 8, 16))], 128 * 4000)
    n = info.n_video
    mism = 0
    for i in range(30000):
        b = rng.uniform(1.0, n - 1.0) if i % 3 else rng.randint(1, n - 2) + rng.random() * 1e-9
        sel = veda.veda_select_query(info, veda.budget(("tiles", b)), veda.budget(("tiles", b)), 64, 1)
        lo, hi, frac = budget.split(b, n)
        k = sel.blocks[0]
        mism += (k.k_lo, k.k_hi, k.frac) != (lo, hi, frac)
    assert mism == 0


def test_ratio_budget_matches_python_arithmetic():
    rng = random.Random(99)
    for _ in range(3000):
        T, H, W = rng.randint(1, 40), rng.randint(1, 60), rng.randint(1, 90)
        seq = T * H * W + rng.randint(0, 300)
        ratio = rng.random() * 1.1
        info = veda.veda_plan_query([(0, (T, H, W), None)], seq)
        sel = veda.veda_select_query(info, veda.budget(("ratio", ratio)),
                                     veda.budget(("ratio", ratio)), 128, 1)
        n = info.n_video
        bud = (ratio, None)
        k = sel.blocks[0]
        if budget.keeps_all(bud):
            assert k.keep_all == 1
            continue
        want = budget.split(budget.per_row(bud, T * H * W, n), n)
        assert (k.k_lo, k.k_hi, k.frac) == want


@pytest.mark.parametrize("bad", [("ratio", -0.5), ("tiles", -1.0)])
def test_select_query_refuses_bad_budget(bad):
    info = veda.veda_plan_query([(0, (4, 16, 16), None)], 1024)
    with pytest.raises(veda.VedaError):
        veda.veda_select_query(info, veda.budget(bad), veda.budget(bad), 64, 1)


def test_select_query_unsupported_head_dim():
    info = veda.veda_plan_query([(0, (4, 16, 16), None)], 1024)
    with pytest.raises(veda.VedaUnsupported):
        veda.veda_select_query(info, veda.budget(("ratio", 0.2)), veda.budget(("ratio", 0.2)), 96, 1)


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # noqa: BLE001
        return False


@pytest.mark.parametrize("grid,seq_len,D,stride_s", [
    ((64, 512, 512), 1 << 24, 64, 64),    # 2^24 rows (2 GiB): past the 24-bit row factor
    ((1, 1, 1), 1, 128, 1 << 23),         # row pitch of 2^24 bytes (one row: tiny extent)
    ((4, 16, 16), 4096, 128, 64),         # rows narrower than head_dim overlap
])
@pytest.mark.parametrize("entry", ["veda_attend_check", "veda_attend"])
def test_attend_refuses_unaddressable_bf16_rows(grid, seq_len, D, stride_s, entry):
    """The bf16 path forms row offsets as 24-bit row x 24-bit pitch in 32 bits;
    layouts outside that are refused on the host: by veda_attend_check, which
    never launches, and by veda_attend before its launch. The dummy aligned
    pointers are never dereferenced; veda_attend itself is only called where
    no GPU is visible, so a regression there could never launch on them."""
    import ctypes as C
    from learned_block_sparse_amd import _lib
    if entry == "veda_attend" and _gpu_visible():
        pytest.skip("calls veda_attend with dummy pointers: CPU-only check")
    if entry == "veda_attend" and not _lib.has_kernels():
        pytest.skip("host-only build of the library")
    lib = _lib.load()
    info = veda.veda_plan_query([(0, grid, None)], seq_len)
    sel = veda.veda_select_query(info, veda.budget(("tiles", 1.0)), veda.budget(("tiles", 1.0)),
                                 D, 1)
    heads = (C.c_int32 * 1)(0)
    dummy = C.c_void_p(1 << 20)
    args = [C.byref(info), C.byref(sel), dummy, dummy, dummy, dummy, dummy, dummy,
            1, stride_s, D, stride_s, D, 1, heads, dummy, dummy]
    st = lib.veda_attend(*args, 0.0, None) if entry == "veda_attend" else \
        lib.veda_attend_check(*args)
    assert st == 2
    assert "bf16 attend needs" in lib.veda_last_error().decode()


def test_attend_check_accepts_a_valid_call_and_names_bad_arguments():
    import ctypes as C
    lib = _lib.load()
    info = veda.veda_plan_query([(0, (4, 16, 16), None)], 1024)
    sel = veda.veda_select_query(info, veda.budget(("tiles", 2.0)), veda.budget(("tiles", 2.0)),
                                 64, 2)
    heads = (C.c_int32 * 2)(0, 1)
    p = C.c_void_p(1 << 20)

    def call(q=p, heads=heads, dtype=1, ss=128, sh=64, total=2, ro=p):
        return lib.veda_attend_check(C.byref(info), C.byref(sel), p, p, q, p, p, p, dtype, ss, sh,
                                     ss, sh, total, heads, ro, p)
    assert call() == 0 and lib.veda_last_error().decode() == ""
    assert call(q=C.c_void_p(0)) == 1 and "q is NULL" in lib.veda_last_error().decode()
    assert call(q=C.c_void_p((1 << 20) + 2)) == 2           # misaligned base
    assert call(total=1) == 1 and "head index 1" in lib.veda_last_error().decode()
    assert call(ro=C.c_void_p(0)) == 1
    assert call(dtype=7) == 1


@pytest.mark.parametrize("name,D", [("padding", 64), ("mid", 128), ("headline", 128)])
def test_int8_workspace_size(name, D):
    """veda_attend_int8's workspace: the int8 codes of every K tile of every
    head (n_heads x n_tiles x 128 x D bytes), then one fp32 scale per tile
    and head, each part rounded up to 256 bytes."""
    wl = workloads.get(name)
    info = veda.veda_plan_query(_spans(wl, wl.head_shapes[0]), wl.seq_len)
    for nh in (1, 3, 24):
        sel = veda.veda_select_query(info, veda.budget(wl.generated), veda.budget(wl.reference),
                                     D, nh)
        up = lambda x: -(-x // 256) * 256  # noqa: E731
        want = up(up(nh * info.n_tiles * 128 * D) + 4 * nh * info.n_tiles)
        assert veda.veda_attend_int8_query(info, sel) == want


def test_int8_refuses_bad_workspace():
    """Too small, NULL or misaligned workspaces are refused on the host before
    anything launches; a head whose codes would reach 2 GiB is unsupported.
    Dummy pointers, never dereferenced: the launching entry point is called
    only where no GPU is visible."""
    import ctypes as C
    info = veda.veda_plan_query([(0, (4, 16, 16), None)], 1024)
    sel = veda.veda_select_query(info, veda.budget(("tiles", 2.0)), veda.budget(("tiles", 2.0)),
                                 64, 2)
    need = veda.veda_attend_int8_query(info, sel)
    big = veda.veda_plan_query([(0, (2048, 64, 128), (1, 8, 16))], 2048 * 64 * 128)
    big_sel = veda.veda_select_query(big, veda.budget(("tiles", 1.0)), veda.budget(("tiles", 1.0)),
                                     128, 1)
    with pytest.raises(veda.VedaUnsupported):
        veda.veda_attend_int8_query(big, big_sel)
    if _gpu_visible() or not _lib.has_kernels():
        pytest.skip("calls veda_attend_int8 with dummy pointers: CPU-only check with kernels")
    lib = _lib.load()
    heads = (C.c_int32 * 2)(0, 1)
    p = C.c_void_p(1 << 20)

    def call(ws=p, nbytes=need):
        return lib.veda_attend_int8(C.byref(info), C.byref(sel), p, p, p, p, p, p, 128, 64, 128,
                                    64, 2, heads, p, p, 0.0, ws, nbytes, None)
    assert call(nbytes=need - 1) == 1 and "workspace smaller" in lib.veda_last_error().decode()
    assert call(ws=C.c_void_p(0)) == 1
    assert call(ws=C.c_void_p((1 << 20) + 8)) == 1 and "aligned" in lib.veda_last_error().decode()


def test_index_lists_and_policy():
    assert veda.parse_index_list("0, 1, 47-49") == {0, 1, 47, 48, 49}
    assert veda.parse_index_list("") == frozenset() and veda.parse_index_list(None) == frozenset()
    assert veda.parse_index_list(" 3 ;5-5 ") == {3, 5}
    for bad in ("a", "4-2", "-1", "1-x"):
        with pytest.raises(veda.VedaError):
            veda.parse_index_list(bad)
    pol = veda.Policy.from_text("0-4, 45-49", "0")
    assert pol.keeps_full(layer=3) and pol.keeps_full(layer=10, step=0)
    assert not pol.keeps_full(layer=10, step=1) and not pol.keeps_full()


def test_full_attention_layers_use_callers_attention_and_count():
    """A call the policy marks for full attention runs the caller's own
    attention (the model keeps it, as the node's full_attention_layers do),
    writes it into `out` when given, and counts as a dense call of 100%
    computed; no libveda entry point is reached (CPU tensors here)."""
    import torch
    S, H, D = 1024, 2, 64
    q = torch.randn(S, H, D)
    pol = veda.Policy.from_text("0-1")
    stats, out = {}, torch.zeros(S, H, D)
    res = veda.attention(q, q, q, [], (0, (4, 16, 16)), [None] * H, None, None,
                         ("sparsity", 0.9), ("sparsity", 0.9), out=out, stats=stats,
                         fallback=lambda a, b, c: a * 2.0, layer=1, policy=pol)
    assert res is out and torch.equal(out, q * 2.0)
    assert stats["dense_calls"] == 1 and stats.get("sparse_calls", 0) == 0
    assert stats["entries"] == stats["dense"] == H * (S / 128) ** 2
    assert "100.0% of full attention" in veda.summary(stats)
    assert veda.receipt(stats).splitlines()[-1] == "Calls: 0 sparse, 1 dense"


def test_attention_unsupported_uses_callers_fallback():
    """A head_dim libveda does not handle is refused on the host before any
    launch; with a fallback the caller's own attention runs, with a warning,
    and the receipt says so; without one the refusal is raised."""
    import torch
    q = torch.zeros(1024, 2, 96)
    args = (q, q, q, [], (0, (4, 16, 16)), [None, None], None, None, ("sparsity", 0.9),
            ("sparsity", 0.9))
    with pytest.raises(veda.VedaUnsupported):
        veda.attention(*args)
    stats = {}
    with pytest.warns(RuntimeWarning):
        out = veda.attention(*args, stats=stats, fallback=lambda q, k, v: "callers-own")
    assert out == "callers-own"
    assert "caller's own attention" in veda.summary(stats)
    # a caller-supplied out receives the fallback's result
    buf = torch.full((1024, 2, 96), 5.0)
    with pytest.warns(RuntimeWarning):
        got = veda.attention(*args, out=buf, fallback=lambda q, k, v: q + 1.0)
    assert got is buf and torch.equal(buf, q + 1.0)


def test_summary_receipt():
    assert veda.summary({"entries": 109, "dense": 1000.0}) == \
        "Attention computed: 10.9% of full attention (89.1% skipped)"
    lines = veda.receipt({"entries": 109, "dense": 1000.0, "sparse_calls": 160,
                          "dense_calls": 40}).splitlines()
    assert lines[0].startswith("Veda done") and lines[2] == "Calls: 160 sparse, 40 dense"


def test_missing_library_fails_loudly(tmp_path):
    """With libveda.so absent, the first call into the package raises and
    names the build step; nothing falls back to another compute path."""
    code = (
        "import learned_block_sparse_amd as veda\n"
        "for call in (lambda: veda.veda_plan_query([(0, (4, 16, 16), None)], 1024),\n"
        "             veda.version):\n"
        "    try:\n"
        "        call()\n"
        "    except RuntimeError as e:\n"
        "        assert 'not found' in str(e) and 'no fallback' in str(e), e\n"
        "    else:\n"
        "        raise SystemExit('no error')\n"
        "print('ok')\n")
    env = dict(os.environ, VEDA_LIBRARY=str(tmp_path / "absent" / "libveda.so"),
               CUDA_VISIBLE_DEVICES="", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
