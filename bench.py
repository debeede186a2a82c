"""Benchmark of one Veda attention layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload headline] [--no-cpu]
                    [--qk bf16|int8]

A step is the whole hot path over the layer: plan (tile packing), select
(pooling, fp64 tile logits, top-k -> CSR tile lists) and attend (tile-skip
attention), with q/k/v already resident in HBM. Timing uses HIP events on the
stream the kernels run on. Prints one JSON line:
  value        kept-tile TFLOP/s of the whole step (kept pairs x 4*128^2*D / step time)
  ms_per_step  ms per layer (plan + select + attend)
  roofline     the attend kernel against MI355X's dense bf16 MFMA peak
  cpu_baseline the CPU oracle on a bounded sample of the same layer, scaled
plus context: attend TFLOP/s over real rows only, and the vendor library's
bf16 GEMM rate measured in the same run (the practical MFMA ceiling).

--qk int8 runs the attend stage with int8 q.k products (veda_attend_int8:
K quantisation pre-pass + attend); its roofline peak is the mixed MFMA rate
of that kernel's work, half its flops in int8 and half (P V) in bf16. A bf16
run also times the int8 attend call alone on the same layer ("int8_qk").
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "kept-tile attention TFLOP/s & ms/layer at 104k tokens, 90% sparse; % MFMA peak"
BF16_PEAK_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 flop/clk/CU (dense bf16 MFMA)
HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 2 * BF16_PEAK_TFLOPS   # dense int8 MFMA: twice the bf16 rate
# Q K^T (half the attend flops) at the int8 rate, P V (the other half) at bf16
MIXED_PEAK_TFLOPS = 1.0 / (0.5 / INT8_PEAK_TOPS + 0.5 / BF16_PEAK_TFLOPS)


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="headline")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--qk", choices=("bf16", "int8"), default="bf16",
                    help="q.k products of the attend stage: bf16 (default) or int8")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run two device copies of MIB MiB (the known-size kernel that "
                         "calibrates the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


# HBM traffic of the attend kernel, from rocprofv3 counter runs recorded in
# these files (see them for the commands and the copy-kernel calibration). It is
# reported only while the kernel source is the one the counters were taken on.
TRAFFIC_FILES = {qk: os.path.join(ROOT, "profiles", f"attend_{name}_headline_traffic.md")
                 for qk, name in (("bf16", "bf16"), ("int8", "i8"))}
_CSRC = os.path.join(ROOT, "learned_block_sparse_amd", "csrc")
KERNEL_SOURCES = {
    "bf16": ("attend.hip", "attend_common.hpp", "kernels.hpp"),
    "int8": ("attend_i8.hip", "attend_i8.hpp", "attend_common.hpp", "kernels.hpp"),
}
KERNEL_NAMES = {"bf16": "attend_bf16_kernel<128>", "int8": "attend_i8_kernel<128>"}


def _kernel_digest(qk):
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[qk]:
        with open(os.path.join(_CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _recorded_traffic(workload, qk="bf16"):
    """Bytes per attend launch from the recorded counters, or None when the
    record is missing, for another workload or kernel, or for another kernel
    source."""
    import re
    try:
        with open(TRAFFIC_FILES[qk]) as f:
            text = f.read()
    except OSError:
        return None
    for m in re.finditer(r"<!-- traffic (\{.*?\}) -->", text):
        rec = json.loads(m.group(1))
        if rec.get("workload") == workload and rec.get("kernel") == KERNEL_NAMES[qk] and \
                rec.get("kernel_sha256") == _kernel_digest(qk):
            return float(rec["bytes_per_launch"])
    return None


def _copy_probe(mib):
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "copies": 2}), flush=True)


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


class Layer:
    """Device buffers and the three stage calls for one workload."""

    def __init__(self, inp):
        import torch
        import learned_block_sparse_amd as veda
        import workloads
        self.veda = veda
        wl = inp.workload
        self.wl = wl
        dev = torch.device("cuda", 0)
        self.t = {}
        for name in ("q", "k", "v"):
            x = getattr(inp, name)
            if wl.dtype == "bf16":
                t = torch.from_numpy(workloads.bf16_bits(x).view(np.int16)).view(torch.bfloat16)
            else:
                t = torch.from_numpy(x)
            self.t[name] = t.to(dev)
        self.out = torch.empty_like(self.t["q"])
        pq = torch.from_numpy(inp.proj_q).to(dev)
        pk = torch.from_numpy(inp.proj_k).to(dev)
        gen, ref = veda.budget(wl.generated), veda.budget(wl.reference)
        tile_refs = not (ref.tiles < 0 and ref.ratio >= 1.0)
        groups = {}
        for h, s in enumerate(wl.head_shapes):
            groups.setdefault(s, []).append(h)
        self.groups = []
        for shape, heads in groups.items():
            spans = [(s, g, None) for s, g in wl.refs] if tile_refs else []
            spans.append((wl.target[0], wl.target[1], shape))
            info = veda.veda_plan_query(spans, wl.seq_len)
            sel = veda.veda_select_query(info, gen, ref, wl.head_dim, len(heads))
            idx = torch.tensor(heads, dtype=torch.long, device=dev)
            g = dict(info=info, sel=sel, heads=heads,
                     perm=torch.empty(info.n_slots, dtype=torch.int32, device=dev),
                     vc=torch.empty(info.n_tiles, dtype=torch.int32, device=dev),
                     ro=torch.empty(info.n_tiles + 1, dtype=torch.int32, device=dev),
                     cols=torch.empty(len(heads) * sel.entries_per_head, dtype=torch.int32, device=dev),
                     ws=torch.empty(sel.workspace_bytes, dtype=torch.uint8, device=dev),
                     ws8=torch.empty(veda.veda_attend_int8_query(info, sel), dtype=torch.uint8,
                                     device=dev) if wl.dtype == "bf16" else None,
                     pq=pq.index_select(0, idx).contiguous(), pk=pk.index_select(0, idx).contiguous())
            self.groups.append(g)
        self.pairs = sum(len(g["heads"]) * g["sel"].entries_per_head for g in self.groups)
        self.flops = self.pairs * 4.0 * 128 * 128 * wl.head_dim

    def real_row_flops(self):
        """Flops over real rows only: sum over kept pairs (a, b) of
        4 * D * valid_count[a] * valid_count[b] (call after select)."""
        import torch
        total = 0.0
        for g in self.groups:
            vc = g["vc"].double()
            ro = g["ro"].long()
            counts = ro[1:] - ro[:-1]
            row_of_entry = torch.repeat_interleave(torch.arange(len(counts), device=vc.device),
                                                   counts)
            cols = g["cols"].view(len(g["heads"]), -1).long()
            per_head = (vc[row_of_entry][None, :] * vc[cols]).sum()
            total += float(per_head) * 4.0 * self.wl.head_dim
        return total

    def plan(self):
        for g in self.groups:
            self.veda.veda_plan(g["info"], g["perm"], g["vc"])

    def select(self):
        v = self.veda
        for g in self.groups:
            v.veda_select(g["info"], g["sel"], g["perm"], g["vc"], self.t["q"], self.t["k"],
                          g["heads"], g["pq"], g["pk"], row_offsets=g["ro"], cols=g["cols"],
                          workspace=g["ws"])

    def attend(self):
        v = self.veda
        for g in self.groups:
            v.veda_attend(g["info"], g["sel"], g["perm"], g["vc"], self.t["q"], self.t["k"],
                          self.t["v"], g["heads"], g["ro"], g["cols"], out=self.out)

    def attend_int8(self):
        v = self.veda
        for g in self.groups:
            v.veda_attend_int8(g["info"], g["sel"], g["perm"], g["vc"], self.t["q"], self.t["k"],
                               self.t["v"], g["heads"], g["ro"], g["cols"], out=self.out,
                               workspace=g["ws8"])


def _gemm_ceiling(n=16384, reps=5):
    """bf16 dense GEMM rate of the vendor library on this GPU (n x n x n,
    fp32 accumulate), the practical MFMA ceiling beside the published peak."""
    import torch
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    return 2.0 * n ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_baseline(inp, layer_pairs, head_dim, seconds):
    """The oracle, as it stands, on a bounded sample of the same layer: pool,
    logits and selection for head 0 (one of H), then exact attention for
    query tiles of head 0 in a seeded order until `seconds` have passed.
    The whole layer's time is extrapolated as H x (head-0 selection) +
    (kept pairs of the layer / kept pairs attended) x (attention time)."""
    from oracle import attention, layer as olayer, selection
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()
                       if p.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001 - report what can be known
        threads = len(os.sched_getaffinity(0))
    wl = inp.workload
    shape = wl.head_shapes[0]
    from oracle import budget as obudget, predictor, tiles as otiles
    gen, ref = obudget.from_request(wl.generated), obudget.from_request(wl.reference)
    t0 = time.perf_counter()
    oshape = otiles.least_padding_shape(wl.target[1]) if shape is None else shape
    lay = olayer.layout_for(wl, oshape, gen, ref)
    t_plan = time.perf_counter() - t0
    t0 = time.perf_counter()
    blocks = selection.column_blocks(lay, gen, ref)
    fq = predictor.pool(inp.q, lay, [0])
    fk = predictor.pool(inp.k, lay, [0])
    sc = predictor.logits(fq, fk, inp.proj_q[[0]], inp.proj_k[[0]])
    kept = selection.select(sc, lay, blocks)
    mask = selection.block_mask(kept, lay)
    t_sel = time.perf_counter() - t0
    order = np.random.default_rng(99).permutation(lay.n_tiles)
    done_pairs, t_att, n_tiles = 0, 0.0, 0
    for a in order:
        t0 = time.perf_counter()
        attention.attend(inp.q, inp.k, inp.v, lay, mask, [0], query_tiles=[a])
        t_att += time.perf_counter() - t0
        done_pairs += int(mask[0, a].sum())
        n_tiles += 1
        if t_att + t_sel >= seconds:
            break
    est = t_plan + wl.n_heads * t_sel + t_att * (layer_pairs / max(1, done_pairs))
    flops = layer_pairs * 4.0 * 128 * 128 * head_dim
    return {
        "value": flops / est / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
        "cpu_model": _cpu_model(),
        "sample": (f"head 0 of {wl.n_heads}: plan + pool + logits + select ({t_sel:.2f} s), then "
                   f"exact fp64 attention for {n_tiles} query tiles ({done_pairs} kept pairs, "
                   f"{t_att:.2f} s); layer time extrapolated to {est:.1f} s"),
        "est_layer_s": est,
    }


def main():
    args = _args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the Veda hot path is single-GPU "
              f"(heads would shard with no exchange); got --gpus {args.gpus}", file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads

    torch.cuda.set_device(0)
    if args.copy_probe:
        _copy_probe(args.copy_probe)
        return
    _log(f"[bench] generating {args.workload}")
    inp = workloads.generate(args.workload)
    wl = inp.workload
    if args.qk == "int8" and wl.dtype != "bf16":
        print("--qk int8 takes a bf16 workload", file=sys.stderr)
        sys.exit(2)
    L = Layer(inp)
    attend = L.attend_int8 if args.qk == "int8" else L.attend
    _log(f"[bench] kept pairs {L.pairs}, {L.flops / 1e12:.3f} TFLOP per layer")

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    # cold plan (first call)
    e0, e1 = ev(), ev()
    e0.record()
    L.plan()
    e1.record()
    torch.cuda.synchronize()
    plan_cold_ms = e0.elapsed_time(e1)

    for _ in range(args.warmup):
        L.plan(); L.select(); attend()
    torch.cuda.synchronize()
    _log("[bench] warmup done")

    marks = []
    t_start, t_stop = ev(), ev()
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(args.steps):
        m = [ev() for _ in range(4)]
        m[0].record(); L.plan()
        m[1].record(); L.select()
        m[2].record(); attend()
        m[3].record()
        marks.append(m)
    t_stop.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_stop)
    ms_step = total_ms / args.steps
    plan_ms = [m[0].elapsed_time(m[1]) for m in marks]
    sel_ms = [m[1].elapsed_time(m[2]) for m in marks]
    att_ms = [m[2].elapsed_time(m[3]) for m in marks]
    att_avg = float(np.mean(att_ms))
    _log(f"[bench] step {ms_step:.3f} ms: plan {np.median(plan_ms):.3f} select "
         f"{np.median(sel_ms):.3f} attend {np.median(att_ms):.3f}")

    attend_tflops = L.flops / (att_avg * 1e-3) / 1e12
    peak = MIXED_PEAK_TFLOPS if args.qk == "int8" else BF16_PEAK_TFLOPS
    real_flops = L.real_row_flops()
    int8_leg = None
    if args.qk == "bf16" and wl.dtype == "bf16":
        # the int8 attend call alone on the same layer and tile lists
        L.attend_int8()
        torch.cuda.synchronize()
        ms8 = []
        for _ in range(args.steps):
            a, b = ev(), ev()
            a.record(); L.attend_int8(); b.record()
            ms8.append((a, b))
        torch.cuda.synchronize()
        ms8 = [a.elapsed_time(b) for a, b in ms8]
        t8 = L.flops / (float(np.mean(ms8)) * 1e-3) / 1e12
        int8_leg = {
            "attend_median_ms": float(np.median(ms8)), "attend_tflops": t8,
            "pct_mixed_peak": 100.0 * t8 / MIXED_PEAK_TFLOPS,
            "mixed_peak_tflops": MIXED_PEAK_TFLOPS,
            "note": "veda_attend_int8 (K quantisation + attend) on the same layer; "
                    "approximate (int8 q.k), not the headline path",
        }
        _log(f"[bench] int8 q.k attend {np.median(ms8):.3f} ms ({t8:.0f} TFLOP/s)")
    gemm = _gemm_ceiling()
    _log(f"[bench] bf16 GEMM ceiling {gemm:.1f} TFLOP/s")
    result = {
        "metric": METRIC,
        "value": L.flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16, q.k int8" if args.qk == "int8" else wl.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: {wl.note}",
            "seq_len": wl.seq_len, "heads": wl.n_heads, "head_dim": wl.head_dim,
            "generated_budget": list(wl.generated), "reference_budget": list(wl.reference),
            "kept_tile_pairs": L.pairs, "tflop_per_layer": L.flops / 1e12,
            "parallelism": "single GPU", "qk": args.qk,
        },
        "stages_ms": {
            "plan_cold": plan_cold_ms,
            "plan_median": float(np.median(plan_ms)),
            "select_median": float(np.median(sel_ms)),
            "attend_median": float(np.median(att_ms)),
            "attend_p10": float(np.percentile(att_ms, 10)),
            "attend_p90": float(np.percentile(att_ms, 90)),
        },
        "attend_tflops": attend_tflops,
        "attend_pct_bf16_peak": 100.0 * attend_tflops / BF16_PEAK_TFLOPS,
        "int8_qk": int8_leg,
        "attend_real_row_tflops": real_flops / (att_avg * 1e-3) / 1e12,
        "gemm_ceiling_tflops": gemm,
        "attend_pct_gemm_ceiling": 100.0 * attend_tflops / gemm,
        "roofline": {
            "bound": "mfma", "achieved": attend_tflops, "peak": peak,
            "unit": "TFLOP/s", "frac": attend_tflops / peak,
            "traffic": _recorded_traffic(wl.name, args.qk),
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu:
        _log("[bench] timing the CPU oracle on a sample")
        result["cpu_baseline"] = _cpu_baseline(inp, L.pairs, wl.head_dim, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
