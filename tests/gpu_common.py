"""Shared helpers of the GPU parity tests: move a workload's inputs to the
device, run libveda's stages through the C ABI, and fetch what the oracle
computes for the same inputs."""
from __future__ import annotations

import sys

import numpy as np

import learned_block_sparse_amd as veda
import workloads
from oracle import budget, layer, selection, tiles

TILE = 128


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(inp, device="cuda"):
    import torch
    wl = inp.workload
    out = {}
    for name in ("q", "k", "v"):
        x = getattr(inp, name)
        if wl.dtype == "bf16":
            t = torch.from_numpy(workloads.bf16_bits(x).view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(np.ascontiguousarray(x))
        out[name] = t.to(device)
    out["proj_q"] = torch.from_numpy(inp.proj_q).to(device)
    out["proj_k"] = torch.from_numpy(inp.proj_k).to(device)
    return out


def group_spans(wl, shape, gen, ref):
    tile_refs = not budget.keeps_all(ref)
    sp = [(s, g, None) for s, g in wl.refs] if tile_refs else []
    sp.append((wl.target[0], wl.target[1], shape))
    return sp


class GpuGroup:
    """One head group run through plan -> select -> attend on the device."""

    def __init__(self, inp, dev, shape, heads, scores_mode=1, oracle_scores=None):
        import torch
        wl = inp.workload
        self.gen = budget.from_request(wl.generated)
        self.ref = budget.from_request(wl.reference)
        oshape = tiles.least_padding_shape(wl.target[1]) if shape is None else shape
        spans = group_spans(wl, oshape, self.gen, self.ref)
        self.info = veda.veda_plan_query(spans, wl.seq_len)
        self.perm, self.vc = veda.veda_plan(self.info)
        self.sel = veda.veda_select_query(self.info, veda.budget(wl.generated),
                                          veda.budget(wl.reference), wl.head_dim, len(heads))
        self.heads = list(heads)
        idx = torch.tensor(self.heads, dtype=torch.long, device=dev["q"].device)
        pq = dev["proj_q"].index_select(0, idx).contiguous()
        pk = dev["proj_k"].index_select(0, idx).contiguous()
        nv = self.info.n_video
        if scores_mode == 2:
            self.scores = torch.from_numpy(np.ascontiguousarray(oracle_scores)).to(dev["q"].device)
        else:
            self.scores = torch.empty((len(heads), nv, nv), dtype=torch.float64,
                                      device=dev["q"].device)
        self.row_offsets, self.cols = veda.veda_select(
            self.info, self.sel, self.perm, self.vc, dev["q"], dev["k"], self.heads, pq, pk,
            scores=self.scores, scores_mode=scores_mode)

    def attend(self, dev, out=None):
        return veda.veda_attend(self.info, self.sel, self.perm, self.vc, dev["q"], dev["k"],
                                dev["v"], self.heads, self.row_offsets, self.cols, out=out)

    def csr(self):
        ro = self.row_offsets.cpu().numpy().astype(np.int64)
        cols = self.cols.cpu().numpy().reshape(len(self.heads), -1)
        return ro, cols


def bf16_half_ulp(x):
    """Half the spacing of bf16 values at |x| (8 significant bits): the most
    that rounding an exact result to bf16 moves it."""
    m, e = np.frexp(np.abs(np.asarray(x, dtype=np.float64)))
    e = np.where(m == 0, -125, e)          # zero: the smallest normal's spacing
    return np.ldexp(1.0, e - 9)


def excess_over_bf16_rounding(got, want):
    """|got - want| beyond the half ulp that rounding the exact `want` to a
    bf16 output may already cost; zero for a correctly rounded result."""
    return np.maximum(0.0, np.abs(got - want) - bf16_half_ulp(want))


def oracle_csr(mask):
    off, cols = selection.tile_lists(mask)
    return off, cols


def near_tie_rows(scores, kept, blocks_params, layout):
    """Rows whose selection could flip under ~1e-12 relative changes: the gap
    between the last kept and the first dropped finite score, relative to the
    row's largest |score|."""
    flagged = []
    H, nv, _ = scores.shape
    for (start, stop, keep_all, lo, hi, frac) in blocks_params:
        if keep_all:
            continue
        for h in range(H):
            for r in range(nv):
                s = scores[h, r, start:stop].copy()
                k = kept[h, r, start:stop]
                if start <= r < stop:
                    s[r - start] = np.inf
                fin = np.isfinite(s)
                if k.all() or (~k).all():
                    continue
                lo_kept = s[k & fin].min() if (k & fin).any() else np.inf
                hi_drop = s[~k].max()
                scale = np.abs(s[fin]).max() if fin.any() else 1.0
                if (lo_kept - hi_drop) <= 1e-12 * max(scale, 1e-300):
                    flagged.append((h, r))
    return flagged
