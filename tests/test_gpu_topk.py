"""GPU qsa_topk against the oracle's selection: ids must match bit for bit."""
import numpy as np
import pytest

import oracle
import qsa_synth
from gpu_util import gpu_topk, upload

pytestmark = pytest.mark.gpu


def _inputs_with_scores(T, pos0, budget, kind, seed, n_cells=None):
    inp = qsa_synth.layer_inputs(T, pos0, seed=seed, budget=budget, n_cells=n_cells,
                                 with_scores=True)
    if kind != "normal":
        inp.scores = qsa_synth.score_rows(T, 2, inp.n_cells, seed, kind=kind, levels=4)
    return inp


@pytest.mark.parametrize("T,pos0,budget,kind", [
    (96, 2050, 2051, "normal"), (32, 2050, 2051, "normal"), (4, 2049, 2051, "normal"),
    (64, 1987, 2051, "normal"), (200, 1900, 2051, "normal"),
    (40, 60, 5, "normal"), (40, 60, 5, "quantized"), (30, 3000, 2051, "quantized"),
    (16, 700, 300, "signed_zero"), (8, 100, 1, "normal"), (8, 5000, 4096, "normal"),
])
def test_topk_matches_oracle(T, pos0, budget, kind):
    inp = _inputs_with_scores(T, pos0, budget, kind, seed=T + pos0)
    ref = oracle.select(T, pos0, budget, inp.scores, 2, inp.n_cells)
    np.testing.assert_array_equal(gpu_topk(inp), ref)


@pytest.mark.parametrize("T,pos0", [(4, 3000), (3, 20000)])
def test_topk_all_equal_and_monotone_rows(T, pos0):
    # at 20,000 cells (the streamed-list kernel) an all-equal row puts every
    # key at the sampled threshold, more than the list holds: the radix and
    # bitmap passes then re-read the row from memory
    B = 2051
    inp = _inputs_with_scores(T, pos0, B, "normal", seed=2)
    N = inp.n_cells
    for s in (np.zeros((T, 2, N), np.float32),
              -np.tile(np.arange(N, dtype=np.float32), (T, 2, 1)),
              np.tile(np.arange(N, dtype=np.float32), (T, 2, 1))):
        inp.scores = s
        np.testing.assert_array_equal(gpu_topk(inp), oracle.select(T, pos0, B, s, 2, N))


def test_topk_scores_row_stride_is_n_cells():
    # n_cells larger than pos0 + T: rows are n_cells apart, cells past n_kv
    # (filled with +inf here) are never selected
    T, pos0, B = 6, 2100, 2051
    inp = _inputs_with_scores(T, pos0, B, "normal", seed=9, n_cells=pos0 + T + 37)
    for t in range(T):
        inp.scores[t, :, pos0 + t + 1:] = np.inf
    np.testing.assert_array_equal(gpu_topk(inp),
                                  oracle.select(T, pos0, B, inp.scores, 2, inp.n_cells))


@pytest.mark.parametrize("kind", ["normal", "quantized"])
def test_topk_rows_longer_than_the_register_tile(kind):
    # rows of more than 512 x 64 cells take the streamed kernel: 3 tokens
    # at pos0 33000 (up to 33,003 cells), normal and tie-heavy scores
    T, pos0, B = 3, 33000, 2051
    inp = _inputs_with_scores(T, pos0, B, kind, seed=17)
    ref = oracle.select(T, pos0, B, inp.scores, 2, inp.n_cells)
    np.testing.assert_array_equal(gpu_topk(inp), ref)


@pytest.mark.parametrize("T,pos0", [(2, 32766), (2, 32767), (2, 16382), (2, 16383), (3, 4093)])
def test_topk_rows_at_register_tile_edges(T, pos0):
    # the longest row exactly fills (pos0 + T = 4096, 16384, 32768 cells) or
    # just passes (16385, 32769) a register tile of 512 threads x 8/32/64
    inp = _inputs_with_scores(T, pos0, 2051, "quantized", seed=pos0)
    ref = oracle.select(T, pos0, 2051, inp.scores, 2, inp.n_cells)
    np.testing.assert_array_equal(gpu_topk(inp), ref)


@pytest.mark.parametrize("kind", ["quantized", "signed_zero", "gap"])
def test_topk_register_rows_with_ties_and_gaps(kind):
    # rows of 20,000..20,003 cells: four score levels, or a gap between the
    # selected scores and a dense rest, stay on the sampled-threshold list;
    # mostly-zero rows put ~19,000 keys at or above the sampled threshold,
    # more than the LDS list holds, so the full register passes run
    T, pos0, B = 4, 20000, 2051
    inp = _inputs_with_scores(T, pos0, B, "normal" if kind == "gap" else kind, seed=77)
    if kind == "gap":
        s = inp.scores
        s[:, :, :B] += np.float32(100.0)  # the first budget cells stand far above the rest
        inp.scores = s
    ref = oracle.select(T, pos0, B, inp.scores, 2, inp.n_cells)
    np.testing.assert_array_equal(gpu_topk(inp), ref)


@pytest.mark.parametrize("pos0,ept", [(12000, 32), (20000, 64)])
def test_topk_rows_whose_sample_holds_the_largest_scores(pos0, ept):
    # The threshold comes from 1024 sampled cells: for s < 16, the 64 cells
    # from 512 i + 64 (s // 2) on, slice i = s * ept / 16 (512 threads,
    # ept slices).  Raising exactly those cells far above the rest puts the
    # sample's rank-r key among them, so fewer than budget cells reach the
    # threshold: the select must fall back (register passes for rows of at
    # most 16,384 cells, passes that re-read the row above) and still give
    # the oracle's ids
    T, B = 3, 2051
    inp = _inputs_with_scores(T, pos0, B, "normal", seed=pos0 + 5)
    s = inp.scores
    for k in range(16):
        c0 = 512 * (k * ept // 16) + 64 * (k // 2)
        s[:, :, c0:c0 + 64] += np.float32(100.0)
    inp.scores = s
    ref = oracle.select(T, pos0, B, inp.scores, 2, inp.n_cells)
    np.testing.assert_array_equal(gpu_topk(inp), ref)
