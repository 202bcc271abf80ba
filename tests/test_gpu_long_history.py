"""A KV history past 2^24 cells per group.

Byte offsets of its cells no longer fit 32 bits (cell * 256 >= 2^32), and
the second group's codes begin 4.3 GB into their array, so the attention
kernels take their 64-bit addressing.  Only the cells some row selects are
drawn (qsa_synth.sparse_history); the device arrays hold zeros elsewhere,
so a gather from a wrong address shows up as a wrong output.  The oracle
attends the same values from a compact copy (the selected cells renumbered
in order), which changes no term of any row.  Three chunk sizes take the
fused call's three row paths: 4 tokens (8 rows, one chunk per piece: the
split kernel), 40 tokens (80 rows: row pieces of 3 chunks on the staged
kernel) and 260 tokens (520 rows: the staged kernel, a row per wavefront).

Selection: page "round 6 track b - qsa flash" (delivered change: the
top-budget cells above budget); attention: page "opus_r9_qsa" (what
changed)."""
import numpy as np
import pytest
import torch

import oracle
import qsa_synth
import quantized_sparse_flash_amd as qsa
from gpu_util import DEV, Guarded, worst_row_rel_l2

N_CELLS = (1 << 24) + 4096


def _compact(h):
    """LayerInputs over the selected cells only, and ids renumbered to them."""
    G = len(h.cells)
    n_u = max(len(c) for c in h.cells)
    pos0 = max(n_u, h.budget)
    n_cells = pos0 + h.T
    D = h.q.shape[2]
    kq = np.zeros((G, n_cells, D), np.int8)
    vq = np.zeros((G, n_cells, D), np.int8)
    ksc = np.zeros((G, n_cells, D // 64), np.float16)
    vsc = np.zeros((G, n_cells, D // 64), np.float16)
    ids = np.empty_like(h.ids)
    for g in range(G):
        n = len(h.cells[g])
        kq[g, :n], vq[g, :n], ksc[g, :n], vsc[g, :n] = h.kq[g], h.vq[g], h.ksc[g], h.vsc[g]
        ids[:, g, :] = np.searchsorted(h.cells[g], h.ids[:, g, :])
    inp = qsa_synth.LayerInputs(T=h.T, pos0=pos0, budget=h.budget, n_cells=n_cells, q=h.q,
                                kq=kq, ksc=ksc, vq=vq, vsc=vsc, scores=None)
    return inp, ids


@pytest.fixture(scope="module", params=[4, 40, 260], ids=lambda t: "T%d" % t)
def history(request):
    T = request.param
    h = qsa_synth.sparse_history(T, N_CELLS - T, N_CELLS)
    assert int(h.ids.max()) >= (1 << 24)
    G = len(h.cells)
    dev = {
        "kq": torch.zeros((G, N_CELLS, 256), dtype=torch.int8, device=DEV),
        "vq": torch.zeros((G, N_CELLS, 256), dtype=torch.int8, device=DEV),
        "ksc": torch.zeros((G, N_CELLS, 4), dtype=torch.float16, device=DEV),
        "vsc": torch.zeros((G, N_CELLS, 4), dtype=torch.float16, device=DEV),
    }
    for g in range(G):
        idx = torch.from_numpy(h.cells[g]).to(DEV)
        for k in ("kq", "vq", "ksc", "vsc"):
            dev[k][g].index_copy_(0, idx, torch.from_numpy(getattr(h, k)[g]).to(DEV))
    dev["q"] = torch.from_numpy(h.q).to(DEV)
    dev["ids"] = torch.from_numpy(h.ids).to(DEV)
    inp, ids = _compact(h)
    ref = oracle.attend(inp, ids)
    yield h, dev, ref
    del dev
    torch.cuda.empty_cache()


@pytest.mark.gpu
def test_fused_rows_past_2_24_cells(history):
    h, dev, ref = history
    T = h.T
    s = qsa.QsaShape(T=T, pos0=h.pos0, n_groups=len(h.cells), budget=h.budget, n_cells=N_CELLS)
    out = Guarded((T, s.n_heads, 256), torch.float16, fill=float("nan"))
    qsa.qsa_flash(s, dev["q"], dev["kq"], dev["ksc"], dev["vq"], dev["vsc"], dev["ids"], out.t)
    got = out.numpy("qsa_flash out").astype(np.float64)
    err = worst_row_rel_l2(got, ref)
    assert err <= 1e-3, "fused, n_cells 2^24 + 4096: worst row rel L2 %.3e" % err


@pytest.mark.gpu
def test_split_and_merge_past_2_24_cells(history):
    h, dev, ref = history
    T = h.T
    s = qsa.QsaShape(T=T, pos0=h.pos0, n_groups=len(h.cells), budget=h.budget, n_cells=N_CELLS)
    part = Guarded((T, s.n_part_chunks, s.n_heads, qsa.PART_STRIDE), torch.float32,
                   fill=float("nan"))
    out = Guarded((T, s.n_heads, 256), torch.float16, fill=float("nan"))
    qsa.qsa_flash(s, dev["q"], dev["kq"], dev["ksc"], dev["vq"], dev["vsc"], dev["ids"], None,
                  part.t)
    qsa.qsa_merge(s, part.t, out.t)
    part.check("qsa_flash part")
    got = out.numpy("qsa_merge out").astype(np.float64)
    err = worst_row_rel_l2(got, ref)
    assert err <= 1e-3, "split + merge, n_cells 2^24 + 4096: worst row rel L2 %.3e" % err
