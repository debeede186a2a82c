"""Veda learned block-sparse attention on MI355X (gfx950).

Python binding over libveda's C ABI (include/veda.h). The functions named
like the C entry points (veda_plan_query, veda_plan, veda_select_query,
veda_select, veda_attend) marshal torch tensors to pointers and the current
HIP stream; `attention` composes them for one layer the way the page
`veda_core.py` (section "one layer") does: per group of heads sharing a tile
box, plan -> select -> attend. PyTorch only supplies device memory and
streams; every step of the path runs in libveda's HIP kernels.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass

from . import _lib
from ._lib import Budget, PlanInfo, SelectInfo, Span, TILE

__all__ = ["VedaError", "VedaUnsupported", "VedaDeviceError", "budget", "summary", "veda_plan_query",
           "veda_plan", "veda_select_query", "veda_select", "veda_attend", "Plan", "plan",
           "attention", "version", "library_path"]


class VedaError(ValueError):
    """A request libveda refused (bad span list, budget or sizes)."""


class VedaUnsupported(VedaError):
    """A valid request outside what the kernels handle (head_dim, alignment)."""


class VedaDeviceError(RuntimeError):
    """A HIP launch or call failed."""


def library_path() -> str:
    return _lib.LIB_PATH


def version() -> str:
    return _lib.load().veda_version().decode()


def _check(status: int):
    if status == _lib.OK:
        return
    msg = _lib.load().veda_last_error().decode()
    if status == _lib.ERR_UNSUPPORTED:
        raise VedaUnsupported(msg)
    if status == _lib.ERR_DEVICE:
        raise VedaDeviceError(msg)
    raise VedaError(msg)


def budget(request) -> Budget:
    """('sparsity', s) | ('ratio', r) | ('tiles', n) -> the C budget record.
    A sparsity s keeps ratio 1.0 - s of the key tiles."""
    kind, value = request
    if kind == "sparsity":
        return Budget(1.0 - float(value), -1.0)
    if kind == "ratio":
        return Budget(float(value), -1.0)
    if kind == "tiles":
        return Budget(-1.0, float(value))
    raise VedaError(f"unknown budget kind {kind!r}")


def _keeps_all(b: Budget) -> bool:
    return b.tiles < 0.0 and b.ratio >= 1.0


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _ptr(t):
    return C.c_void_p(t.data_ptr()) if t is not None else C.c_void_p(0)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return _lib.BF16
    if t.dtype == torch.float32:
        return _lib.F32
    raise VedaUnsupported(f"dtype {t.dtype} (bf16 or float32 only)")


def _check_qkv(*ts):
    t0 = ts[0]
    for t in ts:
        if t.dim() != 3 or not t.is_cuda:
            raise VedaError("q, k, v must be [S, H, D] device tensors")
        if t.stride(2) != 1:
            raise VedaUnsupported("the last (head_dim) axis must be contiguous")
        if t.shape != t0.shape or t.stride() != t0.stride() or t.dtype != t0.dtype:
            raise VedaError("q, k, v must share shape, strides and dtype")


def _heads_array(heads):
    hs = [int(h) for h in heads]
    return (C.c_int32 * len(hs))(*hs), len(hs)


# ------------------------------------------------------------------- plan --
def veda_plan_query(spans, seq_len) -> PlanInfo:
    """spans: [(start, (T, H, W), (t, h, w) or None)] in packed order, the
    target last. None asks for the least-padding box."""
    arr = (Span * max(1, len(spans)))()
    for i, (start, grid, shape) in enumerate(spans):
        arr[i].start = int(start)
        for a in range(3):
            arr[i].grid[a] = int(grid[a])
            arr[i].shape[a] = 0 if shape is None else int(shape[a])
    info = PlanInfo()
    _check(_lib.load().veda_plan_query(arr, len(spans), int(seq_len), C.byref(info)))
    return info


def veda_plan(info: PlanInfo, perm=None, valid_count=None, stream=None, device=None):
    """Builds (perm int32 [n_slots], valid_count int32 [n_tiles]) on the device."""
    import torch
    dev = device or torch.device("cuda", torch.cuda.current_device())
    if perm is None:
        perm = torch.empty(info.n_slots, dtype=torch.int32, device=dev)
    if valid_count is None:
        valid_count = torch.empty(info.n_tiles, dtype=torch.int32, device=dev)
    if perm.numel() < info.n_slots or valid_count.numel() < info.n_tiles:
        raise VedaError("perm / valid_count too small for the plan")
    _check(_lib.load().veda_plan(C.byref(info), _ptr(perm), _ptr(valid_count), _stream(stream)))
    return perm, valid_count


# ----------------------------------------------------------------- select --
def veda_select_query(info: PlanInfo, generated: Budget, reference: Budget, head_dim: int,
                      n_heads: int) -> SelectInfo:
    sel = SelectInfo()
    _check(_lib.load().veda_select_query(C.byref(info), generated, reference, int(head_dim),
                                         int(n_heads), C.byref(sel)))
    return sel


def veda_select(info: PlanInfo, sel: SelectInfo, perm, valid_count, q, k, heads,
                proj_q=None, proj_k=None, scores=None, scores_mode=0, row_offsets=None,
                cols=None, workspace=None, stream=None):
    """Pool, score and select on the device. Returns (row_offsets, cols).
    proj_q / proj_k: float32 [n_heads, 3D, D] device tensors (modes 0, 1).
    scores: float64 [n_heads, n_video, n_video] (written in mode 1, read in 2)."""
    import torch
    dev = perm.device
    harr, nh = _heads_array(heads)
    if nh != sel.n_heads:
        raise VedaError("len(heads) differs from the n_heads given to veda_select_query")
    if row_offsets is None:
        row_offsets = torch.empty(info.n_tiles + 1, dtype=torch.int32, device=dev)
    if cols is None:
        cols = torch.empty(nh * sel.entries_per_head, dtype=torch.int32, device=dev)
    if scores_mode != 2:
        _check_qkv(q, k)
        for p in (proj_q, proj_k):
            if p is None or p.dtype != torch.float32 or not p.is_contiguous() or \
                    tuple(p.shape) != (nh, 3 * sel.head_dim, sel.head_dim):
                raise VedaError("proj_q / proj_k must be contiguous float32 [n_heads, 3D, D]")
        if workspace is None:
            workspace = torch.empty(sel.workspace_bytes, dtype=torch.uint8, device=dev)
        dt, ss, sh, ht = _dtype_code(q), q.stride(0), q.stride(1), q.shape[1]
        ws_bytes = workspace.numel() * workspace.element_size()
    else:
        dt, ss, sh, ht, ws_bytes = _lib.BF16, 0, 0, max(int(h) for h in heads) + 1, 0
    if scores is not None and (scores.dtype != torch.float64 or not scores.is_contiguous()):
        raise VedaError("scores must be contiguous float64")
    _check(_lib.load().veda_select(
        C.byref(info), C.byref(sel), _ptr(perm), _ptr(valid_count),
        _ptr(q) if scores_mode != 2 else None, _ptr(k) if scores_mode != 2 else None, dt,
        ss, sh, ht, harr, _ptr(proj_q), _ptr(proj_k), _ptr(row_offsets), _ptr(cols),
        _ptr(scores), int(scores_mode), _ptr(workspace), ws_bytes, _stream(stream)))
    return row_offsets, cols


# ----------------------------------------------------------------- attend --
def veda_attend(info: PlanInfo, sel: SelectInfo, perm, valid_count, q, k, v, heads,
                row_offsets, cols, out=None, scale=0.0, stream=None):
    """Tile-skip attention; writes every row of the listed heads of `out`
    ([S, H, D], q's dtype; allocated if None) and returns it."""
    import torch
    _check_qkv(q, k, v)
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape or out.dtype != q.dtype or out.stride(2) != 1:
        raise VedaError("out must match q's shape and dtype with a contiguous last axis")
    harr, nh = _heads_array(heads)
    if nh != sel.n_heads:
        raise VedaError("len(heads) differs from the n_heads given to veda_select_query")
    _check(_lib.load().veda_attend(
        C.byref(info), C.byref(sel), _ptr(perm), _ptr(valid_count), _ptr(q), _ptr(k), _ptr(v),
        _ptr(out), _dtype_code(q), q.stride(0), q.stride(1), out.stride(0), out.stride(1),
        q.shape[1], harr, _ptr(row_offsets), _ptr(cols), float(scale), _stream(stream)))
    return out


# ------------------------------------------------------------- one layer --
@dataclass
class Plan:
    """A cached layout for one head group (the page caches layouts per
    geometry, box and whether references are tiled)."""
    info: PlanInfo
    perm: object
    valid_count: object


def plan(spans, seq_len, stream=None, device=None) -> Plan:
    info = veda_plan_query(spans, seq_len)
    perm, vc = veda_plan(info, stream=stream, device=device)
    return Plan(info, perm, vc)


def _head_groups(head_shapes):
    groups = {}
    for h, s in enumerate(head_shapes):
        key = None if s is None else tuple(int(x) for x in s)
        groups.setdefault(key, []).append(h)
    return list(groups.items())


def attention(q, k, v, refs, target, head_shapes, proj_q, proj_k, generated, reference,
              cache=None, out=None, stats=None, stream=None, fallback=None):
    """One layer of Veda attention over q, k, v [S, H, D] (bf16 or float32).

    refs        : [(start, (T, H, W))] reference video spans (packed order)
    target      : (start, (T, H, W)), the generated video, packed last
    head_shapes : per head, the target's tile box or None (least padding)
    proj_q/k    : float32 [H, 3D, D] device tensors
    generated, reference : budget requests, e.g. ('sparsity', 0.9)
    cache       : optional dict holding plans between calls
    stats       : optional dict; gets kept tile pairs ('entries') and the dense
                  count ('dense'), see summary()
    fallback    : optional callable(q, k, v) -> out, the caller's own attention.
                  When libveda refuses the layout (VedaUnsupported: head_dim,
                  alignment, sizes), it is called instead, with a warning: the
                  node described on the comfyui-wiki Veda news pages (Spanish
                  and French editions, section on requirements) reports the
                  problem and lets the model keep its own attention for that
                  run. Without a fallback the error is raised.

    References are tiled with their least-padding box unless the reference
    budget keeps everything, in which case their rows stay global (dense).
    Every host-side check of every head group runs before the first launch.
    Returns out [S, H, D] in q's dtype.
    """
    try:
        return _attention(q, k, v, refs, target, head_shapes, proj_q, proj_k, generated,
                          reference, cache, out, stats, stream)
    except VedaUnsupported as e:
        if fallback is None:
            raise
        import warnings
        warnings.warn(f"veda attention does not support this layout ({e}); "
                      "using the caller's attention", RuntimeWarning, stacklevel=2)
        if stats is not None:
            stats["fallback"] = str(e)
        return fallback(q, k, v)


def _attention(q, k, v, refs, target, head_shapes, proj_q, proj_k, generated, reference,
               cache, out, stats, stream):
    S, H, D = q.shape
    gen, ref = budget(generated), budget(reference)
    tile_refs = not _keeps_all(ref)
    cache = {} if cache is None else cache
    groups = []
    for shape, heads in _head_groups(head_shapes):
        spans = [(s, g, None) for s, g in refs] if tile_refs else []
        spans.append((target[0], target[1], shape))
        info = veda_plan_query(spans, S)
        sel = veda_select_query(info, gen, ref, D, len(heads))
        groups.append((shape, heads, spans, sel))
    import torch
    if out is None:
        out = torch.empty_like(q)
    for shape, heads, spans, sel in groups:
        key = (tuple((int(s), tuple(g)) for s, g in refs), (int(target[0]), tuple(target[1])),
               shape, tile_refs, S, str(q.device))
        if key not in cache:
            cache[key] = plan(spans, S, stream=stream, device=q.device)
        p = cache[key]
        idx = torch.tensor(heads, dtype=torch.long, device=q.device)
        pq = proj_q.index_select(0, idx).contiguous()
        pk = proj_k.index_select(0, idx).contiguous()
        ro, cols = veda_select(p.info, sel, p.perm, p.valid_count, q, k, heads, pq, pk,
                               stream=stream)
        veda_attend(p.info, sel, p.perm, p.valid_count, q, k, v, heads, ro, cols, out=out,
                    stream=stream)
        if stats is not None:
            stats.setdefault("entries", 0)
            stats["entries"] += len(heads) * sel.entries_per_head
            stats.setdefault("dense", 0.0)
            stats["dense"] += len(heads) * float(p.info.n_tiles) ** 2
    return out


def summary(stats) -> str:
    """The per-run receipt of the node's status line (comfyui-wiki Veda news
    pages, the node's output): the share of full attention computed, in tile
    pairs, and the share skipped."""
    if stats.get("fallback"):
        return f"Attention computed by the caller's own attention ({stats['fallback']})"
    dense = stats.get("dense", 0.0)
    share = 100.0 * stats.get("entries", 0) / dense if dense else 0.0
    return f"Attention computed: {share:.1f}% of full attention ({100.0 - share:.1f}% skipped)"
