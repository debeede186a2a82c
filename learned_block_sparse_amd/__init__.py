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

__all__ = ["VedaError", "VedaUnsupported", "VedaDeviceError", "budget", "summary", "receipt",
           "veda_plan_query", "veda_plan", "veda_select_query", "veda_select", "veda_attend",
           "veda_attend_check", "veda_select_static", "veda_teacher", "veda_recall",
           "veda_attend_int8_query", "veda_attend_int8", "Plan", "plan", "Policy", "parse_index_list", "attention",
           "version", "library_path"]


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


def _on_callers_stream(fn):
    """Runs fn with torch's current stream set to its `stream` argument when
    one is given, so that torch's own work for the call (output and workspace
    allocations, the projections' index_select, small copies) is ordered with
    the library's launches on that stream: temporaries are then reused by the
    caching allocator only after the launches that read them."""
    import functools
    import inspect
    pos = list(inspect.signature(fn).parameters).index("stream")

    @functools.wraps(fn)
    def wrapped(*args, **kwargs):
        stream = kwargs.get("stream") if len(args) <= pos else args[pos]
        if stream is None:
            return fn(*args, **kwargs)
        import torch
        with torch.cuda.stream(stream):
            return fn(*args, **kwargs)
    return wrapped


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


@_on_callers_stream
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


@_on_callers_stream
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
        selects = any(not sel.blocks[b].keep_all for b in range(sel.n_blocks))
        if workspace is None and (scores_mode == 1 or selects):
            workspace = torch.empty(sel.workspace_bytes, dtype=torch.uint8, device=dev)
        dt, ss, sh, ht = _dtype_code(q), q.stride(0), q.stride(1), q.shape[1]
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
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


@_on_callers_stream
def veda_select_static(info: PlanInfo, sel: SelectInfo, perm, valid_count, q, k, heads,
                       proj_q, proj_k, row_offsets=None, cols=None, stream=None):
    """veda_select (scores_mode 0) without a workspace: the library's fixed
    device scratch holds the pooled features, projections and logits, a few
    heads at a time (include/veda.h, veda_select_static). For callers that
    cannot allocate; pass row_offsets and cols to allocate nothing at all.
    Calls that overlap on one GPU race on the scratch. Returns
    (row_offsets, cols)."""
    import torch
    dev = perm.device
    harr, nh = _heads_array(heads)
    if nh != sel.n_heads:
        raise VedaError("len(heads) differs from the n_heads given to veda_select_query")
    if row_offsets is None:
        row_offsets = torch.empty(info.n_tiles + 1, dtype=torch.int32, device=dev)
    if cols is None:
        cols = torch.empty(nh * sel.entries_per_head, dtype=torch.int32, device=dev)
    _check_qkv(q, k)
    for p in (proj_q, proj_k):
        if p is None or p.dtype != torch.float32 or not p.is_contiguous() or \
                tuple(p.shape) != (nh, 3 * sel.head_dim, sel.head_dim):
            raise VedaError("proj_q / proj_k must be contiguous float32 [n_heads, 3D, D]")
    _check(_lib.load().veda_select_static(
        C.byref(info), C.byref(sel), _ptr(perm), _ptr(valid_count), _ptr(q), _ptr(k),
        _dtype_code(q), q.stride(0), q.stride(1), q.shape[1], harr, _ptr(proj_q), _ptr(proj_k),
        _ptr(row_offsets), _ptr(cols), _stream(stream)))
    return row_offsets, cols


# ----------------------------------------------------------------- attend --
@_on_callers_stream
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


def veda_attend_int8_query(info: PlanInfo, sel: SelectInfo) -> int:
    """Bytes of device workspace veda_attend_int8 needs for this layout and
    head group."""
    n = C.c_size_t(0)
    _check(_lib.load().veda_attend_int8_query(C.byref(info), C.byref(sel), C.byref(n)))
    return int(n.value)


@_on_callers_stream
def veda_attend_int8(info: PlanInfo, sel: SelectInfo, perm, valid_count, q, k, v, heads,
                     row_offsets, cols, out=None, scale=0.0, workspace=None, stream=None):
    """Tile-skip attention with int8 q.k products (include/veda.h,
    veda_attend_int8): bf16 q, k, v; writes every row of the listed heads of
    `out` (allocated if None) and returns it. `workspace`: a device uint8
    tensor of at least veda_attend_int8_query bytes, allocated if None."""
    import torch
    _check_qkv(q, k, v)
    if q.dtype != torch.bfloat16:
        raise VedaError("veda_attend_int8 takes bf16 q, k, v")
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape or out.dtype != q.dtype or out.stride(2) != 1:
        raise VedaError("out must match q's shape and dtype with a contiguous last axis")
    harr, nh = _heads_array(heads)
    if nh != sel.n_heads:
        raise VedaError("len(heads) differs from the n_heads given to veda_select_query")
    need = veda_attend_int8_query(info, sel)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise VedaError("workspace must be a contiguous device tensor")
    _check(_lib.load().veda_attend_int8(
        C.byref(info), C.byref(sel), _ptr(perm), _ptr(valid_count), _ptr(q), _ptr(k), _ptr(v),
        _ptr(out), q.stride(0), q.stride(1), out.stride(0), out.stride(1), q.shape[1], harr,
        _ptr(row_offsets), _ptr(cols), float(scale), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def veda_attend_check(info: PlanInfo, sel: SelectInfo, perm, valid_count, q, k, v, heads,
                      row_offsets, cols, out):
    """Every check veda_attend makes, on the host, launching nothing; raises
    like veda_attend would."""
    _check_qkv(q, k, v)
    harr, nh = _heads_array(heads)
    if nh != sel.n_heads:
        raise VedaError("len(heads) differs from the n_heads given to veda_select_query")
    _check(_lib.load().veda_attend_check(
        C.byref(info), C.byref(sel), _ptr(perm), _ptr(valid_count), _ptr(q), _ptr(k), _ptr(v),
        _ptr(out), _dtype_code(q), q.stride(0), q.stride(1), out.stride(0), out.stride(1),
        q.shape[1], harr, _ptr(row_offsets), _ptr(cols)))


# ---------------------------------------------------- teacher and recall --
@_on_callers_stream
def veda_teacher(info: PlanInfo, perm, valid_count, q, k, heads, head_dim=None, scale=0.0,
                 teacher=None, stream=None):
    """The max-pooled full-attention teacher map, float32 [n_heads, n_tiles,
    n_tiles] on the device (include/veda.h, veda_teacher)."""
    import torch
    _check_qkv(q, k)
    harr, nh = _heads_array(heads)
    D = q.shape[2] if head_dim is None else int(head_dim)
    n = info.n_tiles
    if teacher is None:
        teacher = torch.empty((nh, n, n), dtype=torch.float32, device=q.device)
    if teacher.dtype != torch.float32 or not teacher.is_contiguous() or \
            teacher.numel() < nh * n * n:
        raise VedaError("teacher must be contiguous float32 [n_heads, n_tiles, n_tiles]")
    _check(_lib.load().veda_teacher(
        C.byref(info), _ptr(perm), _ptr(valid_count), _ptr(q), _ptr(k), _dtype_code(q),
        q.stride(0), q.stride(1), q.shape[1], harr, nh, D, float(scale), _ptr(teacher),
        _stream(stream)))
    return teacher


@_on_callers_stream
def veda_recall(info: PlanInfo, sel: SelectInfo, row_offsets, cols, teacher, recall=None,
                stream=None):
    """Per head and query tile, the teacher distribution's share on the tiles
    of the CSR lists: float32 [n_heads, n_tiles] on the device."""
    import torch
    if recall is None:
        recall = torch.empty((sel.n_heads, info.n_tiles), dtype=torch.float32,
                             device=teacher.device)
    _check(_lib.load().veda_recall(C.byref(info), C.byref(sel), _ptr(row_offsets), _ptr(cols),
                                   _ptr(teacher), _ptr(recall), _stream(stream)))
    return recall


# ------------------------------------------------------------- one layer --
@dataclass
class Plan:
    """A cached layout for one head group (the page caches layouts per
    geometry, box and whether references are tiled)."""
    info: PlanInfo
    perm: object
    valid_count: object


@_on_callers_stream
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


def parse_index_list(text) -> frozenset:
    """'0, 1, 47-49' -> {0, 1, 47, 48, 49}: the node's format for its
    full_attention_layers / full_attention_steps inputs (0-based DiT blocks and
    sampling steps; comfyui-wiki Veda news pages, French and Korean editions,
    the node's input table). Empty or None gives the empty set."""
    if text is None:
        return frozenset()
    if not isinstance(text, str):
        return frozenset(int(x) for x in text)
    out = set()
    for part in text.replace(";", ",").split(","):
        part = part.strip()
        if not part:
            continue
        lo, sep, hi = part.partition("-")
        try:
            a = int(lo)
            b = int(hi) if sep else a
        except ValueError:
            raise VedaError(f"not an index or a range: {part!r}") from None
        if a < 0 or b < a:
            raise VedaError(f"bad range {part!r}: indices are 0-based and ranges ascend")
        out.update(range(a, b + 1))
    return frozenset(out)


@dataclass(frozen=True)
class Policy:
    """Which calls keep full attention: listed DiT blocks (layers) and
    sampling steps, as the node's full_attention_layers and
    full_attention_steps inputs set them."""
    full_attention_layers: frozenset = frozenset()
    full_attention_steps: frozenset = frozenset()

    @classmethod
    def from_text(cls, layers="", steps=""):
        return cls(parse_index_list(layers), parse_index_list(steps))

    def keeps_full(self, layer=None, step=None) -> bool:
        return (layer is not None and layer in self.full_attention_layers) or \
            (step is not None and step in self.full_attention_steps)


_KEEP_ALL = ("ratio", 1.0)


@_on_callers_stream
def attention(q, k, v, refs, target, head_shapes, proj_q, proj_k, generated, reference,
              cache=None, out=None, stats=None, stream=None, fallback=None, layer=None,
              step=None, policy=None, qk="bf16"):
    """One layer of Veda attention over q, k, v [S, H, D] (bf16 or float32).

    refs        : [(start, (T, H, W))] reference video spans (packed order)
    target      : (start, (T, H, W)), the generated video, packed last
    head_shapes : per head, the target's tile box or None (least padding)
    proj_q/k    : float32 [H, 3D, D] device tensors
    generated, reference : budget requests, e.g. ('sparsity', 0.9)
    cache       : optional dict holding plans between calls
    out         : optional [S, H, D] output (q's dtype); allocated if None
    stats       : optional dict accumulating the run's receipt (see receipt()):
                  'entries' tile pairs computed, 'dense' the full-attention
                  count (S/128)^2 per head, 'sparse_calls', 'dense_calls'
    fallback    : optional callable(q, k, v) -> out, the caller's own attention.
                  When libveda refuses the layout (VedaUnsupported: head_dim,
                  alignment, sizes), it is called instead, with a warning: the
                  node described on the comfyui-wiki Veda news pages (Spanish
                  and French editions, section on requirements) reports the
                  problem and lets the model keep its own attention for that
                  run. Without a fallback the error is raised.
    layer, step, policy : with a Policy that lists this layer or step, the
                  call keeps full attention: the caller's `fallback` when one
                  is given (the model's own attention), else libveda's
                  kernels with every tile kept, which is exact dense
                  attention. It counts as a dense call in the receipt.
    qk          : "bf16" (default) or "int8": the q.k products of sparse
                  calls in int8 (veda_attend_int8; bf16 q, k, v only). Dense
                  calls keep bf16 products.

    References are tiled with their least-padding box unless the reference
    budget keeps everything, in which case their rows stay global (dense).
    Every host-side check of every head group, the attend limits included,
    runs before the first launch, so a refusal leaves the device untouched.
    Returns out [S, H, D] in q's dtype.
    """
    dense = policy is not None and policy.keeps_full(layer, step)
    if dense:
        generated = reference = _KEEP_ALL
    try:
        if dense and fallback is not None:
            res = _into(out, fallback(q, k, v))
        else:
            res = _attention(q, k, v, refs, target, head_shapes, proj_q, proj_k, generated,
                             reference, cache, out, None if dense else stats, stream,
                             "bf16" if dense else qk)
    except VedaUnsupported as e:
        if fallback is None:
            raise
        import warnings
        warnings.warn(f"veda attention does not support this layout ({e}); "
                      "using the caller's attention", RuntimeWarning, stacklevel=2)
        if stats is not None:
            stats["fallback"] = str(e)
        return _into(out, fallback(q, k, v))
    if stats is not None:
        key = "dense_calls" if dense else "sparse_calls"
        stats[key] = stats.get(key, 0) + 1
        if dense:
            full = q.shape[1] * (q.shape[0] / TILE) ** 2
            stats["entries"] = stats.get("entries", 0) + full
            stats["dense"] = stats.get("dense", 0.0) + full
    return res


def _into(out, res):
    """The caller's own attention result, written into `out` when one was given."""
    if out is None:
        return res
    out.copy_(res)
    return out


def _attention(q, k, v, refs, target, head_shapes, proj_q, proj_k, generated, reference,
               cache, out, stats, stream, qk="bf16"):
    import torch
    S, H, D = q.shape
    if qk not in ("bf16", "int8"):
        raise VedaError(f"qk must be 'bf16' or 'int8', not {qk!r}")
    if qk == "int8" and q.dtype != torch.bfloat16:
        raise VedaUnsupported("int8 q.k products take bf16 q, k, v")
    gen, ref = budget(generated), budget(reference)
    tile_refs = not _keeps_all(ref)
    cache = {} if cache is None else cache
    if out is None:
        out = torch.empty_like(q)
    # host side of every group first: layouts, budgets, buffers, attend limits
    groups = []
    ws_bytes = 0
    for shape, heads in _head_groups(head_shapes):
        spans = [(s, g, None) for s, g in refs] if tile_refs else []
        spans.append((target[0], target[1], shape))
        key = (tuple((int(s), tuple(g)) for s, g in refs), (int(target[0]), tuple(target[1])),
               shape, tile_refs, S, str(q.device))
        p = cache.get(key)
        if p is None:
            info = veda_plan_query(spans, S)
            p = Plan(info, torch.empty(info.n_slots, dtype=torch.int32, device=q.device),
                     torch.empty(info.n_tiles, dtype=torch.int32, device=q.device))
            p.built = False
        sel = veda_select_query(p.info, gen, ref, D, len(heads))
        ro = torch.empty(p.info.n_tiles + 1, dtype=torch.int32, device=q.device)
        cols = torch.empty(len(heads) * sel.entries_per_head, dtype=torch.int32, device=q.device)
        veda_attend_check(p.info, sel, p.perm, p.valid_count, q, k, v, heads, ro, cols, out)
        if qk == "int8":
            ws_bytes = max(ws_bytes, veda_attend_int8_query(p.info, sel))
        groups.append((key, p, heads, sel, ro, cols))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device) if qk == "int8" else None
    for key, p, heads, sel, ro, cols in groups:
        if not getattr(p, "built", True):
            veda_plan(p.info, p.perm, p.valid_count, stream=stream)
            p.built = True
            cache[key] = p
        idx = torch.tensor(heads, dtype=torch.long, device=q.device)
        pq = proj_q.index_select(0, idx).contiguous()
        pk = proj_k.index_select(0, idx).contiguous()
        veda_select(p.info, sel, p.perm, p.valid_count, q, k, heads, pq, pk, row_offsets=ro,
                    cols=cols, stream=stream)
        if qk == "int8":
            veda_attend_int8(p.info, sel, p.perm, p.valid_count, q, k, v, heads, ro, cols,
                             out=out, workspace=ws, stream=stream)
        else:
            veda_attend(p.info, sel, p.perm, p.valid_count, q, k, v, heads, ro, cols, out=out,
                        stream=stream)
        if stats is not None:
            stats["entries"] = stats.get("entries", 0) + len(heads) * sel.entries_per_head
            # full attention: (S / 128)^2 tile pairs per head (page `veda_core.py`,
            # section "one layer", the run's stats), whatever the padding
            stats["dense"] = stats.get("dense", 0.0) + len(heads) * (S / TILE) ** 2
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


def receipt(stats, kernel="HIP bf16 MFMA (gfx950)") -> str:
    """The run's receipt: the kernel that ran, the share line of summary(),
    and the count of sparse and dense (full-attention) calls, as the Vflash
    guide's Veda receipts report them."""
    lines = [f"Veda done \u00b7 {kernel}", summary(stats)]
    sp, dn = stats.get("sparse_calls", 0), stats.get("dense_calls", 0)
    if sp or dn:
        lines.append(f"Calls: {sp} sparse, {dn} dense")
    return "\n".join(lines)
