"""qsa_score against the oracle (the reading of "round 27 track b - qsa prep
and merge", decision and correctness: a score per visible cell from the
token's index query and the cell's pooled key).

Scores are compared over whole tensors with the bound fp32 recursive
summation with fused multiply-adds guarantees, index_dim * 2^-24 * sum_d
|q_d p_d| per element (first order; the factor 1.01 absorbs the rest).
Every element the kernel must not write (rows under budget, cells past the
token's n_kv) is pre-filled with a sentinel that must survive.  End to end,
the GPU's fp32 scores feed qsa_topk on the GPU and the oracle's selection on
the host: the ids must agree bit for bit, and the attention over them must
meet the usual output bar."""
import numpy as np
import pytest
import torch

import oracle
import qsa_synth
import quantized_sparse_flash_amd as qsa
from gpu_util import DEV, Guarded, gpu_flash, shape_of, upload, worst_row_rel_l2

SENTINEL = np.float32(-12345.5)


def _gpu_scores(T, pos0, qidx, pooled, budget=qsa_synth.BUDGET):
    G, n_cells, D = pooled.shape
    s = qsa.QsaShape(T=T, pos0=pos0, n_groups=G, budget=budget, n_cells=n_cells)
    out = Guarded((T, G, n_cells), torch.float32, fill=float(SENTINEL))
    qsa.qsa_score(s, torch.from_numpy(qidx).to(DEV), torch.from_numpy(pooled).to(DEV), out.t)
    return out.numpy("qsa_score scores")


def _check_scores(T, pos0, D, n_cells=None, budget=qsa_synth.BUDGET, seed=5):
    qidx, pooled = qsa_synth.score_inputs(T, pos0, D, seed, n_cells=n_cells)
    got = _gpu_scores(T, pos0, qidx, pooled, budget)
    ref = oracle.score(T, pos0, budget, qidx, pooled)
    written = ~np.isnan(ref)
    assert np.all(got[~written] == SENTINEL), "an element outside the scored rows was written"
    # the first-order fp32 bound, from |q p| summed in fp64 (test arithmetic)
    absdot = np.einsum("tgd,gcd->tgc", np.abs(qidx).astype(np.float64),
                       np.abs(pooled).astype(np.float64))
    bound = 1.01 * D * 2.0 ** -24 * absdot + 1e-30
    err = np.abs(got.astype(np.float64) - ref)
    bad = written & (err > bound)
    assert not bad.any(), "T=%d pos0=%d D=%d: %d scores past the fp32 bound (worst %.3e)" % (
        T, pos0, D, int(bad.sum()), float(np.max(np.where(written, err / bound, 0))))


@pytest.mark.gpu
@pytest.mark.parametrize("T,pos0,D,spare", [(96, 2050, 4, 0), (32, 2050, 4, 0), (96, 2050, 64, 0),
                                            (33, 3000, 256, 777), (96, 1984, 8, 0),
                                            (200, 1900, 4, 1)])
def test_scores_match_oracle_within_fp32_bound(T, pos0, D, spare):
    _check_scores(T, pos0, D, n_cells=pos0 + T + spare)


@pytest.mark.gpu
def test_scores_long_context_whole_tensor():
    # the long-context workload's shape: T=1984 at pos0 30000, four values per cell
    _check_scores(1984, 30000, 4)


@pytest.mark.gpu
def test_no_row_above_budget_writes_nothing():
    qidx, pooled = qsa_synth.score_inputs(64, 0, 4)
    got = _gpu_scores(64, 0, qidx, pooled)
    assert np.all(got == SENTINEL)


@pytest.mark.gpu
@pytest.mark.parametrize("T,pos0", [(96, 2050), (200, 1900)])
def test_score_topk_flash_end_to_end(T, pos0):
    inp = qsa_synth.layer_inputs(T, pos0, with_scores=False)
    qidx, pooled = qsa_synth.score_inputs(T, pos0, 4, n_cells=inp.n_cells)
    s = shape_of(inp)
    scores = Guarded((T, s.n_groups, s.n_cells), torch.float32, fill=0.0)
    qsa.qsa_score(s, torch.from_numpy(qidx).to(DEV), torch.from_numpy(pooled).to(DEV), scores.t)
    ids = Guarded((T, s.n_groups, s.budget), torch.int32, fill=-7)
    qsa.qsa_topk(s, scores.t, ids.t)
    gpu_scores = scores.numpy("qsa_score scores")
    gpu_ids = ids.numpy("qsa_topk ids")
    # the same fp32 scores decide the selection on both sides
    want_ids = oracle.select(T, pos0, s.budget, gpu_scores, s.n_groups, s.n_cells)
    assert np.array_equal(gpu_ids, want_ids)
    out = gpu_flash(inp, gpu_ids, dev=upload(inp))
    ref = oracle.attend(inp, want_ids)
    err = oracle.rel_l2(out, ref)
    assert err <= 1e-3, "end to end rel L2 %.3e" % err
    assert worst_row_rel_l2(out, ref) <= 4e-3
