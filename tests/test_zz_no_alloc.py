"""qsa_flash_noalloc (library-held scratch, no workspace argument) against
qsa_flash with a caller workspace, on two calls in a row of which the
second is smaller (the scratch keeps the first call's images; the second
must not read them): the same bytes when qsa_flash's whole workspace fits
the scratch (both calls then take the same kernels), otherwise the same
output within the oracle's bar (the scratch holds the chunk images, but a
split route whose whole workspace it cannot hold leaves those rows to the
row kernel); and the oracle's bar in every case.  The last pair has no
token under budget: only the row-piece records use the scratch."""
import numpy as np
import pytest
import torch

import oracle
import qsa_synth
import quantized_sparse_flash_amd as qsa
from gpu_util import Guarded, shape_of, upload, worst_row_rel_l2

pytestmark = pytest.mark.gpu


def _noalloc(inp, ids, dev):
    s = shape_of(inp)
    idt = None if ids is None else torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda()
    out = Guarded((s.T, s.n_heads, s.head_dim), torch.float16, fill=float("nan"))
    qsa.qsa_flash_noalloc(s, dev["q"], dev["kq"], dev["ksc"], dev["vq"], dev["vsc"], idt, out.t)
    return out.numpy("qsa_flash_noalloc out").astype(np.float64)


def _with_workspace(inp, ids, dev):
    s = shape_of(inp)
    idt = None if ids is None else torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda()
    out = Guarded((s.T, s.n_heads, s.head_dim), torch.float16, fill=float("nan"))
    ws = torch.empty(max(qsa.qsa_flash_workspace_bytes(s), 1), dtype=torch.uint8, device="cuda")
    qsa.qsa_flash(s, dev["q"], dev["kq"], dev["ksc"], dev["vq"], dev["vsc"], idt, out.t,
                  workspace=ws)
    return out.numpy("qsa_flash out").astype(np.float64)


@pytest.mark.parametrize("cases", [((1984, 0, 3), (512, 0, 4)), ((200, 1900, 1), (33, 0, 2)),
                                   ((96, 2050, 5), (32, 2050, 6))])
def test_noalloc_matches_workspace_call_twice(cases):
    for T, pos0, layer in cases:       # the second call is the smaller one
        inp = qsa_synth.layer_inputs(T, pos0, layer=layer)
        ids = None
        if inp.scores is not None:
            ids = oracle.select(T, pos0, inp.budget, inp.scores, 2, inp.n_cells)
        dev = upload(inp)
        got = _noalloc(inp, ids, dev)
        full = _with_workspace(inp, ids, dev)
        if qsa.qsa_flash_workspace_bytes(shape_of(inp)) <= qsa.NOALLOC_SCRATCH_BYTES:
            np.testing.assert_array_equal(got, full)
        else:
            assert oracle.rel_l2(got, full) <= 1e-3
            assert worst_row_rel_l2(got, full) <= 4e-3
        ref = oracle.attend(inp, ids)
        assert oracle.rel_l2(got, ref) <= 1e-3
        assert worst_row_rel_l2(got, ref) <= 4e-3
