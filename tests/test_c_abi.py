"""include/veda.h from plain C: a C11 program (tests/c_abi_host.c) built with
gcc against the in-tree libveda.so sees the same struct layout as the ctypes
binding and gets the same layouts and budget splits from the host-only calls
as the binding and the oracle. No kernel is launched."""
import ctypes as C
import os
import shutil
import subprocess

import pytest

import learned_block_sparse_amd as veda
from learned_block_sparse_amd import _lib
from oracle import tiles
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.fixture(scope="module")
def c_program(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None or not os.path.isdir(os.path.join(ROCM, "include", "hip")):
        pytest.skip("gcc or the HIP headers are not available")
    if not os.path.exists(_lib.LIB_PATH) or not _lib.has_kernels():
        pytest.skip("needs the in-tree libveda.so")
    exe = str(tmp_path_factory.mktemp("cabi") / "c_abi_host")
    libdir = os.path.dirname(_lib.LIB_PATH)
    subprocess.run([gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-isystem", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c_abi_host.c"), "-o", exe, f"-L{libdir}",
                    "-l:" + os.path.basename(_lib.LIB_PATH), f"-Wl,-rpath,{libdir}"],
                   check=True, capture_output=True, text=True)
    return exe


def _run(exe, spec):
    r = subprocess.run([exe], input=spec, capture_output=True, text=True, check=True, timeout=60)
    return dict(line.split("=", 1) for line in r.stdout.splitlines())


def _spec(wl, shape, n_heads):
    gen, ref = veda.budget(wl.generated), veda.budget(wl.reference)
    lines = [f"seq_len {wl.seq_len}"]
    for s, g in wl.refs:
        lines.append(f"span {s} {g[0]} {g[1]} {g[2]} 0 0 0")
    box = shape or (0, 0, 0)
    t = wl.target
    lines.append(f"span {t[0]} {t[1][0]} {t[1][1]} {t[1][2]} {box[0]} {box[1]} {box[2]}")
    lines.append(f"budget {gen.ratio!r} {gen.tiles!r} {ref.ratio!r} {ref.tiles!r}")
    lines.append(f"head {n_heads} {wl.head_dim}")
    return "\n".join(lines) + "\n"


def test_struct_layout_matches_the_binding(c_program):
    out = _run(c_program, "")
    assert out["version"] == veda.version()
    for cname, ctype in (("veda_span", _lib.Span), ("veda_budget", _lib.Budget),
                         ("veda_plan_info", _lib.PlanInfo), ("veda_block", _lib.Block),
                         ("veda_select_info", _lib.SelectInfo)):
        assert int(out[f"sizeof.{cname}"]) == C.sizeof(ctype), cname
        for key, value in out.items():
            if key.startswith(f"offset.{cname}."):
                field = key.split(".", 2)[2]
                assert int(value) == getattr(ctype, field).offset, (cname, field)


@pytest.mark.parametrize("name", ["tiny", "padding", "mid", "headline", "long"])
def test_host_calls_from_c_match_binding_and_oracle(c_program, name):
    wl = workloads.get(name)
    for shape in sorted(set(wl.head_shapes), key=str):
        heads = [h for h, s in enumerate(wl.head_shapes) if s == shape]
        out = _run(c_program, _spec(wl, shape, len(heads)))
        assert out["plan_status"] == "0" and out["select_status"] == "0", out
        spans = [(s, g, None) for s, g in wl.refs] + [(wl.target[0], wl.target[1], shape)]
        info = veda.veda_plan_query(spans, wl.seq_len)
        sel = veda.veda_select_query(info, veda.budget(wl.generated), veda.budget(wl.reference),
                                     wl.head_dim, len(heads))
        for f in ("n_slots", "n_tiles", "n_video", "n_ref", "n_global", "ref_tokens",
                  "target_tokens", "global_rows"):
            assert int(out[f]) == getattr(info, f), f
        for f in ("n_blocks", "widest", "entries_per_head", "workspace_bytes"):
            assert int(out[f]) == getattr(sel, f), f
        for b in range(sel.n_blocks):
            blk = sel.blocks[b]
            want = f"{blk.start},{blk.stop},{blk.keep_all},{blk.k_lo},{blk.k_hi}"
            got = out[f"block{b}"].rsplit(",", 1)
            assert got[0] == want and float(got[1]) == blk.frac, (b, out[f"block{b}"])
        # the oracle's layout of the same spans (boxes resolved the same way)
        oshape = tiles.least_padding_shape(wl.target[1]) if shape is None else shape
        ospans = [(s, g, tiles.least_padding_shape(g)) for s, g in wl.refs]
        ospans.append((wl.target[0], wl.target[1], oshape))
        lay = tiles.build_layout(ospans, wl.seq_len)
        assert (int(out["n_tiles"]), int(out["n_video"]), int(out["n_global"])) == \
            (lay.n_tiles, lay.n_video, lay.n_global)
        for i, (_, _, s) in enumerate(ospans):
            assert out[f"span{i}.shape"] == ",".join(str(x) for x in s)


def test_refusal_from_c_sets_the_error_text(c_program):
    # two spans that overlap: refused on the host with a reason
    out = _run(c_program, "seq_len 4096\nspan 0 1 16 8 1 16 8\nspan 64 1 16 8 1 16 8\n"
                          "budget 0.5 -1 0.5 -1\nhead 1 128\n")
    assert out["plan_status"] == str(_lib.ERR_INVALID)
    assert out["plan_error"]


def _build_layer_program(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc is not available")
    exe = str(tmp_path / "c_abi_layer")
    libdir = os.path.dirname(_lib.LIB_PATH)
    subprocess.run([gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-isystem", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c_abi_layer.c"), "-o", exe, f"-L{libdir}",
                    "-l:" + os.path.basename(_lib.LIB_PATH), f"-L{os.path.join(ROCM, 'lib')}",
                    "-lamdhip64", f"-Wl,-rpath,{libdir}"],
                   check=True, capture_output=True, text=True)
    return exe


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["padding", "mid"])
def test_layer_from_a_c_program_matches_the_binding(tmp_path, name):
    """A C program that allocates its own device buffers and calls veda_plan,
    veda_select and veda_attend (tests/c_abi_layer.c) writes the same output,
    bit for bit, as the Python binding's one-call layer on the same inputs."""
    import numpy as np
    import torch
    exe = _build_layer_program(tmp_path)
    wl = workloads.get(name)
    assert wl.dtype == "bf16" and set(wl.head_shapes) == {None} and not wl.refs
    inp = workloads.generate(wl)
    for n in "qkv":
        workloads.bf16_bits(getattr(inp, n)).tofile(tmp_path / f"{n}.bin")
    np.ascontiguousarray(inp.proj_q, dtype=np.float32).tofile(tmp_path / "pq.bin")
    np.ascontiguousarray(inp.proj_k, dtype=np.float32).tofile(tmp_path / "pk.bin")
    (tmp_path / "layer.txt").write_text(_spec(wl, None, wl.n_heads))
    print(f"[c-abi] {name}: running the C program", flush=True)
    r = subprocess.run([exe, str(tmp_path)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    got = np.fromfile(tmp_path / "out.bin", dtype=np.uint16).reshape(wl.seq_len, wl.n_heads,
                                                                        wl.head_dim)
    dev = {n: torch.from_numpy(workloads.bf16_bits(getattr(inp, n)).view(np.int16))
           .view(torch.bfloat16).cuda() for n in "qkv"}
    want = veda.attention(dev["q"], dev["k"], dev["v"], wl.refs, wl.target, wl.head_shapes,
                          torch.from_numpy(inp.proj_q).cuda(), torch.from_numpy(inp.proj_k).cuda(),
                          wl.generated, wl.reference)
    torch.cuda.synchronize()
    want = want.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want)
