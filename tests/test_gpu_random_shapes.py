"""Seeded random shapes through the selection, fused, no-alloc and split +
merge paths, against the oracle: 64 draws with 1-3 KV groups and budgets
up to 2051, and 32 wider ones with up to 8 groups and budgets up to 8192
(where the identity prefix's images exceed the no-alloc scratch, that call
must refuse with QSA_ERR_TOO_LARGE).  T, pos0, budget, the number of KV groups
and spare history cells are drawn so that the calls take every route
(tiled blocks with and without split pieces, every token split, split rows
after tiled tokens, the row kernel) and meet ragged chunk, block and budget
edges.  The bar is the same as everywhere: ids bit-exact, outputs within
relative L2 1e-3 (worst row 4e-3) of the oracle."""
import numpy as np
import pytest
import torch

import oracle
import qsa_synth
import quantized_sparse_flash_amd as qsa
from gpu_util import Guarded, gpu_flash, gpu_split_merge, gpu_topk, shape_of, upload, \
    worst_row_rel_l2

pytestmark = pytest.mark.gpu

MAX_VISITS = 600_000  # (token, group, cell) visits per case: the oracle takes well under 1 s


def _visits(T, pos0, budget, G):
    n = np.minimum(pos0 + np.arange(T) + 1, budget)
    return int(n.sum()) * G


def _cases(n=64, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        G = int(rng.choice([1, 2, 2, 2, 3]))
        budget = int(rng.choice([7, 64, 65, 130, 500, 1000, 2051, 2051]))
        T = int(rng.integers(1, 260))
        kind = int(rng.integers(0, 3))
        if kind == 0:    # under budget where T allows it
            pos0 = int(rng.integers(0, max(1, budget - T + 1)))
        elif kind == 1:  # the budget crossed inside the chunk
            pos0 = max(0, budget - int(rng.integers(1, T + 1)))
        else:            # every token above budget
            pos0 = budget + int(rng.integers(0, 3000))
        spare = int(rng.choice([0, 0, 17, 300]))
        if _visits(T, pos0, budget, G) <= MAX_VISITS:
            out.append((len(out), T, pos0, budget, G, spare))
    return out


def _check(got, ref, what):
    assert np.all(np.isfinite(got)), what
    assert oracle.rel_l2(got, ref) <= 1e-3, what
    assert worst_row_rel_l2(got, ref) <= 4e-3, what


def _wide_cases(n=32, seed=101):
    """Wider draws: up to 8 KV groups, budgets from 1 to 8192 (identity
    prefixes up to 128 chunks), chunks up to 699 tokens."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        G = int(rng.choice([1, 2, 4, 5, 8]))
        budget = int(rng.choice([1, 63, 64, 129, 777, 2051, 4096, 8192]))
        T = int(rng.integers(1, 700))
        kind = int(rng.integers(0, 3))
        if kind == 0:
            pos0 = int(rng.integers(0, max(1, budget - T + 1)))
        elif kind == 1:
            pos0 = max(0, budget - int(rng.integers(1, T + 1)))
        else:
            pos0 = budget + int(rng.integers(0, 5000))
        spare = int(rng.choice([0, 5, 1000]))
        if _visits(T, pos0, budget, G) <= 1_500_000:
            out.append((1000 + len(out), T, pos0, budget, G, spare))
    return out


@pytest.mark.parametrize("case,T,pos0,budget,G,spare", _cases() + _wide_cases())
def test_random_shape(case, T, pos0, budget, G, spare):
    inp = qsa_synth.layer_inputs(T, pos0, layer=case, seed=77, budget=budget,
                                 n_cells=pos0 + T + spare, n_groups=G)
    dev = upload(inp)
    ids = None
    if inp.scores is not None:
        ids = oracle.select(T, pos0, budget, inp.scores, G, inp.n_cells)
        np.testing.assert_array_equal(gpu_topk(inp, dev), ids)
    ref = oracle.attend(inp, ids)
    _check(gpu_flash(inp, ids, dev), ref, "qsa_flash")

    s = shape_of(inp)
    idt = None if ids is None else torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda()
    out = Guarded((s.T, s.n_heads, s.head_dim), torch.float16, fill=float("nan"))
    images = G * -(-min(pos0 + T, budget) // qsa.CHUNK) * 65536 if pos0 < budget else 0
    if images <= qsa.NOALLOC_SCRATCH_BYTES:
        qsa.qsa_flash_noalloc(s, dev["q"], dev["kq"], dev["ksc"], dev["vq"], dev["vsc"], idt,
                              out.t)
        _check(out.numpy("qsa_flash_noalloc out").astype(np.float64), ref, "qsa_flash_noalloc")
    else:  # the identity prefix's chunk images exceed the static scratch
        with pytest.raises(qsa.QsaError) as e:
            qsa.qsa_flash_noalloc(s, dev["q"], dev["kq"], dev["ksc"], dev["vq"], dev["vsc"], idt,
                                  out.t)
        assert e.value.status == qsa.QSA_ERR_TOO_LARGE

    _check(gpu_split_merge(inp, ids, dev), ref, "split + merge")
