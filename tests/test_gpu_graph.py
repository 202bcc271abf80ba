"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed.  Every replay must write the same bytes as the same calls run
eagerly (the kernels are deterministic), with other eager work, including
an eager qsa_flash_noalloc on another shape that rewrites the library's
static scratch, and a clobbering fill of every output between replays.
No entry point allocates or records a memset, so capturing them needs
nothing else: the counters of the split paths start at zero because a
kernel of the same call clears them or because the previous call left them
at zero."""
import numpy as np
import pytest
import torch

import qsa_synth
import quantized_sparse_flash_amd as qsa
from gpu_util import DEV, shape_of, upload

pytestmark = pytest.mark.gpu

REPLAYS = 3
_INT_VIEW = {torch.float16: torch.int16, torch.float32: torch.int32, torch.int32: torch.int32,
             torch.int8: torch.int8}
_CLOBBER = {torch.float16: float("nan"), torch.float32: float("nan"), torch.int32: -7,
            torch.int8: 99}


def _bits(t):
    return t.view(_INT_VIEW[t.dtype])


def _other_work():
    """Eager work between replays: a no-alloc call of another shape (it
    rewrites the static scratch a captured no-alloc call also uses) and a
    plain torch kernel."""
    inp = qsa_synth.layer_inputs(64, 0, layer=5)
    d = upload(inp)
    s = shape_of(inp)
    out = torch.empty((s.T, s.n_heads, s.head_dim), dtype=torch.float16, device=DEV)
    qsa.qsa_flash_noalloc(s, d["q"], d["kq"], d["ksc"], d["vq"], d["vsc"], None, out)
    torch.randn(1 << 20, device=DEV).mul_(3.0)


def _check_replays(run, outs):
    """run() eagerly for the reference, then captured once and replayed
    REPLAYS times, each after other work and a clobber of every output."""
    for o in outs:
        o.fill_(_CLOBBER[o.dtype])
    run()
    torch.cuda.synchronize()
    ref = [_bits(o).clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()  # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for r in range(REPLAYS):
        _other_work()
        for o in outs:
            o.fill_(_CLOBBER[o.dtype])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, want) in enumerate(zip(outs, ref)):
            same = torch.equal(_bits(o), want)
            assert same, "replay %d: output %d differs from the eager call" % (r, i)


def _workspace(s):
    n = qsa.qsa_flash_workspace_bytes(s)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=DEV)


def _ids_out(s):
    ids = torch.empty((s.T, s.n_groups, s.budget), dtype=torch.int32, device=DEV)
    out = torch.empty((s.T, s.n_heads, s.head_dim), dtype=torch.float16, device=DEV)
    return ids, out


@pytest.mark.parametrize("T,pos0", [(96, 0), (512, 0), (1984, 0)])
def test_graph_fused_under_budget(T, pos0):
    inp = qsa_synth.layer_inputs(T, pos0, layer=1)
    d = upload(inp)
    s = shape_of(inp)
    ws = _workspace(s)
    _, out = _ids_out(s)

    def run():
        qsa.qsa_flash(s, d["q"], d["kq"], d["ksc"], d["vq"], d["vsc"], None, out, workspace=ws)

    _check_replays(run, [out])


@pytest.mark.parametrize("T,pos0", [(96, 2050), (32, 2050), (200, 1900), (300, 4000)])
def test_graph_topk_then_fused(T, pos0):
    """Top-k then the fused call: every token split (96 and 32 tokens
    crossing the budget), tiled tokens in pieces plus split rows (200 at
    1900), and the row kernel (600 rows above budget)."""
    inp = qsa_synth.layer_inputs(T, pos0, layer=2)
    d = upload(inp)
    s = shape_of(inp)
    ws = _workspace(s)
    ids, out = _ids_out(s)

    def run():
        qsa.qsa_topk(s, d["scores"], ids)
        qsa.qsa_flash(s, d["q"], d["kq"], d["ksc"], d["vq"], d["vsc"], ids, out, workspace=ws)

    _check_replays(run, [ids, out])


def test_graph_score_topk_flash_chain():
    """Selection scores, top-k and attention as one captured chain."""
    T, pos0 = 96, 2050
    inp = qsa_synth.layer_inputs(T, pos0, layer=3)
    d = upload(inp)
    s = shape_of(inp)
    qidx, pooled = qsa_synth.score_inputs(T, pos0, 4, n_cells=s.n_cells)
    qd = torch.from_numpy(qidx).to(DEV)
    pd = torch.from_numpy(pooled).to(DEV)
    scores = torch.empty((s.T, s.n_groups, s.n_cells), dtype=torch.float32, device=DEV)
    ws = _workspace(s)
    ids, out = _ids_out(s)

    def run():
        qsa.qsa_score(s, qd, pd, scores)
        qsa.qsa_topk(s, scores, ids)
        qsa.qsa_flash(s, d["q"], d["kq"], d["ksc"], d["vq"], d["vsc"], ids, out, workspace=ws)

    _check_replays(run, [ids, out])


def test_graph_prepare_then_attend():
    inp = qsa_synth.layer_inputs(1024, 0, layer=4)
    d = upload(inp)
    s = shape_of(inp)
    ws = _workspace(s)
    _, out = _ids_out(s)

    def run():
        qsa.qsa_flash_prepare(s, d["kq"], d["ksc"], d["vq"], d["vsc"], workspace=ws)
        qsa.qsa_flash_attend(s, d["q"], d["kq"], d["ksc"], d["vq"], d["vsc"], None, out,
                             workspace=ws)

    _check_replays(run, [out])


@pytest.mark.parametrize("T,pos0", [(96, 0), (1984, 0), (200, 1900), (96, 2050)])
def test_graph_noalloc(T, pos0):
    """The no-alloc call, whose scratch the eager work between replays
    overwrites with another shape's images."""
    inp = qsa_synth.layer_inputs(T, pos0, layer=6)
    d = upload(inp)
    s = shape_of(inp)
    ids, out = _ids_out(s)
    if inp.scores is not None:
        qsa.qsa_topk(s, d["scores"], ids)
        torch.cuda.synchronize()
    idt = ids if inp.scores is not None else None

    def run():
        qsa.qsa_flash_noalloc(s, d["q"], d["kq"], d["ksc"], d["vq"], d["vsc"], idt, out)

    _check_replays(run, [out])


@pytest.mark.parametrize("T,pos0", [(4, 8192), (8, 30000), (1, 512)])
def test_graph_decode_split_and_merge(T, pos0):
    inp = qsa_synth.layer_inputs(T, pos0, layer=7)
    d = upload(inp)
    s = shape_of(inp)
    ids, out = _ids_out(s)
    part = torch.empty((s.T, s.n_part_chunks, s.n_heads, qsa.PART_STRIDE), dtype=torch.float32,
                       device=DEV)
    idt = ids if inp.scores is not None else None

    def run():
        if idt is not None:
            qsa.qsa_topk(s, d["scores"], ids)
        qsa.qsa_flash(s, d["q"], d["kq"], d["ksc"], d["vq"], d["vsc"], idt, None, part)
        qsa.qsa_merge(s, part, out)

    _check_replays(run, [part, out])


def test_graph_quantize():
    x = torch.from_numpy(qsa_synth.kv_rows(3000, seed=11)).to(DEV)
    codes = torch.empty(x.shape, dtype=torch.int8, device=DEV)
    scales = torch.empty((x.shape[0], 4), dtype=torch.float16, device=DEV)

    def run():
        qsa.qsa_quantize(x, codes, scales)

    _check_replays(run, [codes, scales])
