"""GPU split mode (qsa_flash with part) and qsa_merge against the oracle."""
import numpy as np
import pytest

import oracle
import qsa_synth
from gpu_util import gpu_flash, gpu_merge, gpu_topk, upload, worst_row_rel_l2

pytestmark = pytest.mark.gpu


def _ids(inp):
    if inp.scores is None:
        return None
    return oracle.select(inp.T, inp.pos0, inp.budget, inp.scores, 2, inp.n_cells)


def test_decode_merge_workload():
    # 4 tokens at position 8192: each token's 2051 selected cells in 33
    # chunks; split flash then merge, against exact attention
    inp = qsa_synth.layer_inputs(4, 8192)
    ids = _ids(inp)
    dev = upload(inp)
    np.testing.assert_array_equal(gpu_topk(inp, dev), ids)
    part = gpu_flash(inp, ids, dev, split=True)
    assert part.shape == (4, 33, 24, 258)
    merged = gpu_merge(inp, part)
    ref = oracle.attend(inp, ids)
    assert oracle.rel_l2(merged, ref) <= 1e-3
    assert worst_row_rel_l2(merged, ref) <= 4e-3


@pytest.mark.parametrize("T,pos0", [(4, 8192), (96, 0), (33, 2040), (8, 63), (2, 64)])
def test_split_records_match_oracle_partials(T, pos0):
    inp = qsa_synth.layer_inputs(T, pos0, seed=11)
    ids = _ids(inp)
    part = gpu_flash(inp, ids, split=True)
    m, l, o = oracle.partials(inp, ids, chunk=64)
    nch = oracle.chunk_counts(T, pos0, inp.budget)
    for t in range(T):
        k = nch[t]
        # written records: finite; records past the token's chunks untouched
        assert np.all(np.isfinite(part[t, :k]))
        assert np.all(np.isnan(part[t, k:]))
        gm, gl, go = part[t, :k, :, 256], part[t, :k, :, 257], part[t, :k, :, :256]
        # m_k is a max of scores computed from K rounded once to fp16: the
        # per-score error has sigma ~ 0.0625 * 16 * |q||k| * 2^-11/sqrt(3)
        # ~ 2e-4 on these inputs, so 3e-3 absolute is ~15 sigma
        np.testing.assert_allclose(gm, m[t, :k], rtol=0, atol=3e-3)
        # l and o are relative to m: compare o/l, and l e^m
        assert oracle.rel_l2(go / gl[..., None], o[t, :k] / l[t, :k, :, None]) <= 1e-3
        np.testing.assert_allclose(gl * np.exp(gm), l[t, :k] * np.exp(m[t, :k]), rtol=2e-3)


def test_merge_of_oracle_records():
    # merge kernel alone: the oracle's fp32-packed records in, fp16 out
    inp = qsa_synth.layer_inputs(8, 30000, seed=3)
    ids = _ids(inp)
    m, l, o = oracle.partials(inp, ids, chunk=64)
    part = oracle.pack_part(m, l, o)
    nch = oracle.chunk_counts(8, 30000, inp.budget)
    ref = oracle.merge(part, nch)
    got = gpu_merge(inp, part)
    assert oracle.rel_l2(got, ref) <= 5e-4      # fp16 output rounding only
    assert worst_row_rel_l2(got, ref) <= 2e-3


@pytest.mark.parametrize("pos,ntok", [(0, 1), (1, 2), (63, 4), (64, 8), (512, 1), (2047, 4),
                                      (2048, 2), (2050, 8), (30000, 1)])
def test_split_then_merge_equals_exact(pos, ntok):
    # the pages' decode positions x token counts, as (pos0, T)
    inp = qsa_synth.layer_inputs(ntok, pos, seed=pos + ntok)
    ids = _ids(inp)
    dev = upload(inp)
    if ids is not None:
        np.testing.assert_array_equal(gpu_topk(inp, dev), ids)
    merged = gpu_merge(inp, gpu_flash(inp, ids, dev, split=True))
    fused = gpu_flash(inp, ids, dev)
    ref = oracle.attend(inp, ids)
    assert oracle.rel_l2(merged, ref) <= 1e-3
    assert oracle.rel_l2(fused, ref) <= 1e-3
