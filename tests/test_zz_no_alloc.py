"""veda_select_static, the selection entry point that allocates nothing
(its scratch is a fixed device array), against veda_select with a caller's
workspace: the same row offsets and tile lists, bit for bit, on two calls in
a row through the C ABI, the second on a smaller layer (the scratch then
holds the first call's leftovers), a clear refusal of a layer whose single
head needs more scratch than the array holds, and the layer's three calls
captured into a HIP graph and replayed."""
import ctypes as C

import numpy as np
import pytest

import workloads
from gpu_common import log, to_device

torch = pytest.importorskip("torch")
import learned_block_sparse_amd as veda  # noqa: E402
from learned_block_sparse_amd import _lib  # noqa: E402

pytestmark = pytest.mark.gpu


def _groups(wl):
    g = {}
    for h, s in enumerate(wl.head_shapes):
        g.setdefault(s, []).append(h)
    return list(g.items())


def _both(name):
    inp = workloads.generate(name)
    wl = inp.workload
    dev = to_device(inp)
    gen, ref = veda.budget(wl.generated), veda.budget(wl.reference)
    for shape, heads in _groups(wl):
        spans = [(s, g, None) for s, g in wl.refs] + [(wl.target[0], wl.target[1], shape)]
        info = veda.veda_plan_query(spans, wl.seq_len)
        perm, vc = veda.veda_plan(info)
        sel = veda.veda_select_query(info, gen, ref, wl.head_dim, len(heads))
        idx = torch.tensor(heads, device="cuda")
        pq, pk = dev["proj_q"][idx].contiguous(), dev["proj_k"][idx].contiguous()
        ro_a, cols_a = veda.veda_select(info, sel, perm, vc, dev["q"], dev["k"], heads, pq, pk)
        ro_b = torch.full_like(ro_a, -7)
        cols_b = torch.full_like(cols_a, -7)
        log(f"[no-alloc] {name} shape={shape} heads={len(heads)} "
            f"scratch per head {sel.workspace_bytes // len(heads)} B")
        veda.veda_select_static(info, sel, perm, vc, dev["q"], dev["k"], heads, pq, pk,
                                row_offsets=ro_b, cols=cols_b)
        torch.cuda.synchronize()
        assert torch.equal(ro_a, ro_b), name
        assert torch.equal(cols_a, cols_b), name


def test_select_static_matches_select_two_calls():
    _both("headline")       # 24 heads, several chunks through the scratch
    _both("padding")        # smaller, after it


def test_select_static_refuses_a_head_beyond_the_scratch():
    # 2,752 video tiles at head_dim 64: one head's logits (61 MB), pooled
    # features and projections come to 71.9 MB, past the 64 MiB array
    grid, box = (8, 64, 688), (1, 16, 8)
    S = grid[0] * grid[1] * grid[2]
    info = veda.veda_plan_query([(0, grid, box)], S)
    sel = veda.veda_select_query(info, veda.budget(("ratio", 0.05)),
                                 veda.budget(("ratio", 0.05)), 64, 1)
    assert sel.workspace_bytes > _lib.STATIC_SCRATCH_BYTES
    q = torch.zeros(S, 1, 64, dtype=torch.bfloat16, device="cuda")
    perm, vc = veda.veda_plan(info)
    pq = torch.zeros(1, 192, 64, device="cuda")
    with pytest.raises(veda.VedaUnsupported, match="static scratch"):
        veda.veda_select_static(info, sel, perm, vc, q, q, [0], pq, pq)


def test_graph_capture_replays_plan_select_attend():
    """The caller this entry point exists for: plan, veda_select_static and
    veda_attend captured into one HIP graph (every buffer made before the
    capture; the library itself allocates, copies and clears nothing), then
    replayed three times with eager work and synchronisation between the
    replays. Every replay's layout, tile lists and output equal the eager
    calls' bit for bit."""
    inp = workloads.generate("padding")
    wl = inp.workload
    dev = to_device(inp)
    q, k, v = dev["q"], dev["k"], dev["v"]
    gen, ref = veda.budget(wl.generated), veda.budget(wl.reference)
    shape, heads = _groups(wl)[0]
    spans = [(s, g, None) for s, g in wl.refs] + [(wl.target[0], wl.target[1], shape)]
    info = veda.veda_plan_query(spans, wl.seq_len)
    sel = veda.veda_select_query(info, gen, ref, wl.head_dim, len(heads))
    idx = torch.tensor(heads, device="cuda")
    pq, pk = dev["proj_q"][idx].contiguous(), dev["proj_k"][idx].contiguous()
    perm_e, vc_e = veda.veda_plan(info)
    ro_e, cols_e = veda.veda_select_static(info, sel, perm_e, vc_e, q, k, heads, pq, pk)
    out_e = veda.veda_attend(info, sel, perm_e, vc_e, q, k, v, heads, ro_e, cols_e)
    torch.cuda.synchronize()
    perm, vc = torch.empty_like(perm_e), torch.empty_like(vc_e)
    ro, cols = torch.empty_like(ro_e), torch.empty_like(cols_e)
    out = torch.empty_like(out_e)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        veda.veda_plan(info, perm, vc)
        veda.veda_select_static(info, sel, perm, vc, q, k, heads, pq, pk, row_offsets=ro,
                                cols=cols)
        veda.veda_attend(info, sel, perm, vc, q, k, v, heads, ro, cols, out=out)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (perm, vc, ro, cols):
            t.fill_(-5)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        log(f"[graph] replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(perm, perm_e) and torch.equal(vc, vc_e), rep
        assert torch.equal(ro, ro_e) and torch.equal(cols, cols_e), rep
        assert torch.equal(out[:, heads], out_e[:, heads]), rep
