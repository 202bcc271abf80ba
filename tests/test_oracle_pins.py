"""Pins of the fp64 oracle to things other than itself (CPU only).

Each test checks the oracle against an independent formulation: a dense
numpy brute force with explicit masks, torch's scaled_dot_product_attention
(CPU, fp64), numpy's stable argsort, closed forms and invariants.  A
plausible mistake in the oracle -- a wrong scale, a wrong scale block, an
off-by-one in the visible cells, a wrong tie rule, a dropped merge factor --
fails at least one of them.
"""
import numpy as np
import pytest
import torch

import oracle
import qsa_synth


def _tiny(T, pos0, budget, seed=1, D=64, G=2, HPG=3, n_cells=None, scores="normal"):
    inp = qsa_synth.layer_inputs(T, pos0, seed=seed, budget=budget, n_groups=G,
                                 heads_per_group=HPG, head_dim=D, n_cells=n_cells,
                                 with_scores=True)
    if scores == "quantized":
        inp.scores = qsa_synth.score_rows(T, G, inp.n_cells, seed, kind="quantized", levels=3)
    return inp


# ---------------------------------------------------------------- selection

def _argsort_select(s, n, B):
    """Library pin: numpy stable argsort of -s (ties keep index order)."""
    if n <= B:
        return np.concatenate([np.arange(n), -np.ones(B - n, dtype=np.int64)])
    order = np.argsort(-s[:n].astype(np.float64), kind="stable")[:B]
    return np.sort(order)


@pytest.mark.parametrize("T,pos0,B,kind", [(8, 0, 5, "normal"), (8, 10, 5, "quantized"),
                                           (16, 30, 7, "normal"), (6, 3, 1, "quantized"),
                                           (4, 2049, 2051, "normal")])
def test_select_matches_stable_argsort(T, pos0, B, kind):
    G, N = 2, pos0 + T
    s = qsa_synth.score_rows(T, G, N, 3, kind=kind, levels=4)
    ids = oracle.select(T, pos0, B, s, G, N)
    for t in range(T):
        n = pos0 + t + 1
        for g in range(G):
            np.testing.assert_array_equal(ids[t, g], _argsort_select(s[t, g], n, B))


def test_select_rank_formula_bruteforce():
    # rank_c = #{s > s_c} + #{c' < c, s_c' = s_c}; selected iff rank_c < B
    T, pos0, B, G = 5, 9, 6, 2
    N = pos0 + T
    s = qsa_synth.score_rows(T, G, N, 11, kind="quantized", levels=2)
    ids = oracle.select(T, pos0, B, s, G, N)
    for t in range(T):
        n = pos0 + t + 1
        for g in range(G):
            row = s[t, g, :n]
            sel = [c for c in range(n)
                   if sum(row > row[c]) + sum(row[:c] == row[c]) < B]
            np.testing.assert_array_equal(ids[t, g], sel)


def test_select_special_cases():
    T, pos0, B, G = 3, 20, 8, 1
    N = pos0 + T
    n_last = pos0 + T
    equal = np.zeros((T, G, N), np.float32)
    ids = oracle.select(T, pos0, B, equal, G, N)
    np.testing.assert_array_equal(ids[-1, 0], np.arange(B))      # all ties: lowest ids
    neg = -np.tile(np.arange(N, dtype=np.float32), (T, G, 1))
    np.testing.assert_array_equal(oracle.select(T, pos0, B, neg, G, N)[-1, 0], np.arange(B))
    pos = np.tile(np.arange(N, dtype=np.float32), (T, G, 1))
    np.testing.assert_array_equal(oracle.select(T, pos0, B, pos, G, N)[-1, 0],
                                  np.arange(n_last - B, n_last))
    # scaling by 2 (exact in fp32) and adding an integer to integer scores
    # (exact) never changes the selection
    q = qsa_synth.score_rows(T, G, N, 5, kind="quantized", levels=5)
    base = oracle.select(T, pos0, B, q, G, N)
    np.testing.assert_array_equal(oracle.select(T, pos0, B, q * 2, G, N), base)
    np.testing.assert_array_equal(oracle.select(T, pos0, B, q + 7, G, N), base)


def test_select_signed_zero_is_a_tie():
    T, pos0, B, G = 2, 40, 10, 2
    N = pos0 + T
    s = qsa_synth.score_rows(T, G, N, 8, kind="signed_zero")
    ids = oracle.select(T, pos0, B, s, G, N)
    flipped = np.where(s == 0, -s, s).astype(np.float32)          # swap +0 and -0
    np.testing.assert_array_equal(oracle.select(T, pos0, B, flipped, G, N), ids)
    for t in range(T):
        for g in range(G):
            np.testing.assert_array_equal(ids[t, g], _argsort_select(s[t, g], pos0 + t + 1, B))


def test_identity_rows_ignore_scores_and_budget_edges():
    # n = pos0+t+1 <= budget -> identity; budget 2051 edge: 2051 identity,
    # 2052 drops exactly one cell
    T, pos0, B, G = 4, 2048, 2051, 1
    N = pos0 + T
    s = qsa_synth.score_rows(T, G, N, 2, kind="normal")
    ids = oracle.select(T, pos0, B, s, G, N)
    np.testing.assert_array_equal(ids[0, 0], np.concatenate([np.arange(2049), [-1, -1]]))
    np.testing.assert_array_equal(ids[2, 0], np.arange(2051))     # n = 2051
    assert np.all(ids[3, 0] >= 0) and len(np.unique(ids[3, 0])) == B
    dropped = set(range(2052)) - set(ids[3, 0].tolist())
    assert dropped == {int(np.argmin(s[3, 0, :2052]))}


# ------------------------------------------------------------ attention

@pytest.mark.parametrize("T,pos0,B,kind", [(8, 0, 5, "normal"), (6, 10, 5, "normal"),
                                           (5, 7, 4, "quantized"), (8, 0, 100, "normal"),
                                           (3, 16, 1, "normal")])
def test_attend_matches_dense_bruteforce(T, pos0, B, kind):
    inp = _tiny(T, pos0, B, seed=T + pos0, scores=kind)
    ids = oracle.select(T, pos0, B, inp.scores, 2, inp.n_cells)
    got = oracle.attend(inp, ids)
    ref, mask = oracle.dense_reference(inp, inp.scores)
    # the brute-force mask selects the same cells
    for t in range(T):
        for g in range(2):
            sel = ids[t, g][ids[t, g] >= 0]
            np.testing.assert_array_equal(np.nonzero(mask[t, g])[0], sel)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("T,pos0,D,HPG", [(8, 0, 256, 12), (5, 11, 128, 2), (1, 0, 64, 1)])
def test_identity_equals_library_sdpa(T, pos0, D, HPG):
    # under budget the path is plain causal softmax attention: torch's SDPA
    # on the dequantised K/V (fp64, CPU) with an explicit visibility mask
    G = 2
    inp = qsa_synth.layer_inputs(T, pos0, seed=4, n_groups=G, heads_per_group=HPG,
                                 head_dim=D, budget=4096)
    got = oracle.attend(inp, None)
    k = torch.from_numpy(inp.kq.astype(np.float64)) * \
        torch.from_numpy(inp.ksc.astype(np.float64)).repeat_interleave(64, dim=2)
    v = torch.from_numpy(inp.vq.astype(np.float64)) * \
        torch.from_numpy(inp.vsc.astype(np.float64)).repeat_interleave(64, dim=2)
    q = torch.from_numpy(inp.q.astype(np.float64)).permute(1, 0, 2)  # [H][T][D]
    kh = k.repeat_interleave(HPG, dim=0)                               # [H][N][D]
    vh = v.repeat_interleave(HPG, dim=0)
    N = inp.n_cells
    mask = torch.arange(N)[None, :] <= (pos0 + torch.arange(T))[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(q[None], kh[None], vh[None],
                                                           attn_mask=mask)[0]
    np.testing.assert_allclose(got, ref.permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-13)


def test_single_visible_cell_returns_its_value():
    # token 0 at pos0 0 sees one cell: softmax over one cell gives o = v_0
    inp = qsa_synth.layer_inputs(3, 0, seed=9)
    out = oracle.attend(inp, None)
    for g in range(2):
        v0 = inp.vq[g, 0].astype(np.float64) * np.repeat(inp.vsc[g, 0].astype(np.float64), 64)
        for j in range(12):
            np.testing.assert_allclose(out[0, 12 * g + j], v0, rtol=1e-15, atol=0)


def test_zero_key_scales_give_the_mean_value():
    # all scores 0 -> uniform weights -> o = mean of the selected V rows
    T, pos0, B = 6, 20, 9
    inp = _tiny(T, pos0, B, seed=3, D=128, HPG=2)
    inp.ksc[:] = 0
    ids = oracle.select(T, pos0, B, inp.scores, 2, inp.n_cells)
    out = oracle.attend(inp, ids)
    for t in range(T):
        for g in range(2):
            sel = ids[t, g][ids[t, g] >= 0]
            v = inp.vq[g, sel].astype(np.float64) * \
                np.repeat(inp.vsc[g, sel].astype(np.float64), 64, axis=1)
            for j in range(2):
                np.testing.assert_allclose(out[t, 2 * g + j], v.mean(axis=0), rtol=1e-12,
                                           atol=1e-15)


def test_scaling_and_permutation_invariants():
    T, pos0, B = 5, 30, 12
    inp = _tiny(T, pos0, B, seed=6, D=128, HPG=3)
    ids = oracle.select(T, pos0, B, inp.scores, 2, inp.n_cells)
    base = oracle.attend(inp, ids)
    inp2 = _tiny(T, pos0, B, seed=6, D=128, HPG=3)
    inp2.vsc = (inp2.vsc.astype(np.float32) * 2).astype(np.float16)   # exact doubling
    np.testing.assert_allclose(oracle.attend(inp2, ids), 2 * base, rtol=1e-14, atol=0)
    perm = ids.copy()
    rng = np.random.default_rng(0)
    for t in range(T):
        for g in range(2):
            perm[t, g] = rng.permutation(perm[t, g])
    np.testing.assert_allclose(oracle.attend(inp, perm), base, rtol=1e-12, atol=1e-14)


def test_identity_rows_never_read_ids():
    # poisoned ids (-1) for under-budget tokens change nothing
    T, pos0, B = 6, 0, 4
    inp = _tiny(T, pos0, B, seed=2)
    ids = oracle.select(T, pos0, B, inp.scores, 2, inp.n_cells)
    base = oracle.attend(inp, ids)
    poisoned = ids.copy()
    for t in range(T):
        if pos0 + t + 1 <= B:
            poisoned[t] = -1
    np.testing.assert_array_equal(oracle.attend(inp, poisoned), base)


# -------------------------------------------------------- split and merge

@pytest.mark.parametrize("chunk", [1, 7, 64, 4096])
def test_merge_of_partials_equals_unsplit(chunk):
    T, pos0, B = 6, 70, 90
    inp = _tiny(T, pos0, B, seed=12, D=128, HPG=3)
    ids = oracle.select(T, pos0, B, inp.scores, 2, inp.n_cells)
    full = oracle.attend(inp, ids)
    m, l, o = oracle.partials(inp, ids, chunk=chunk)
    part = oracle.pack_part(m, l, o)
    merged = oracle.merge(part, oracle.chunk_counts(T, pos0, B, chunk))
    # fp32 records: relative rounding ~1e-7
    assert oracle.rel_l2(merged, full) < 2e-7
    np.testing.assert_allclose(merged, full, rtol=2e-5, atol=2e-7)


def test_single_chunk_merges_to_o_over_l_and_order_is_irrelevant():
    T, pos0, B = 4, 0, 64
    inp = _tiny(T, pos0, B, seed=13, D=64, HPG=2)
    m, l, o = oracle.partials(inp, None, chunk=64)
    part = oracle.pack_part(m, l, o)
    merged = oracle.merge(part, oracle.chunk_counts(T, pos0, B, 64))
    np.testing.assert_allclose(merged, o[:, 0] / l[:, 0, :, None], rtol=1e-6)
    # permuting chunk records does not change the merge
    T2, pos02, B2 = 3, 300, 300
    inp2 = _tiny(T2, pos02, B2, seed=14, D=64, HPG=2)
    ids2 = oracle.select(T2, pos02, B2, inp2.scores, 2, inp2.n_cells)
    m2, l2, o2 = oracle.partials(inp2, ids2, chunk=64)
    part2 = oracle.pack_part(m2, l2, o2)
    nch = oracle.chunk_counts(T2, pos02, B2, 64)
    base = oracle.merge(part2, nch)
    shuffled = part2.copy()
    for t in range(T2):
        p = np.random.default_rng(t).permutation(nch[t])
        shuffled[t, :nch[t]] = part2[t, p]
    np.testing.assert_allclose(oracle.merge(shuffled, nch), base, rtol=1e-12)


def test_partials_chunk_max_and_sum_definitions():
    # m_k is the chunk maximum of the scaled scores, l_k the sum of exp(s - m_k):
    # checked against the brute-force score matrix of one row
    T, pos0, B = 1, 130, 200
    inp = _tiny(T, pos0, B, seed=15, D=64, HPG=1)
    m, l, o = oracle.partials(inp, None, chunk=64)
    k = inp.kq.astype(np.float64) * np.repeat(inp.ksc.astype(np.float64), 64, axis=2)
    for h in range(2):
        s = (k[h] @ inp.q[0, h].astype(np.float64)) / 8.0           # 1/sqrt(64)
        s = s[:pos0 + 1]
        for kk in range(3):
            blk = s[64 * kk:64 * kk + 64]
            assert m[0, kk, h] == pytest.approx(blk.max(), rel=1e-14)
            assert l[0, kk, h] == pytest.approx(np.exp(blk - blk.max()).sum(), rel=1e-13)


# ---- selection scores (the reading of "round 27 track b - qsa prep
# and merge": qidx . pooled per cell)

def test_score_agrees_with_a_python_sum():
    """Every score of the rows above budget equals the dot product summed
    term by term in Python floats; spare cells past n_kv stay unwritten."""
    T, pos0, budget, D = 5, 40, 16, 12
    n_cells = pos0 + T + 5
    rng = np.random.default_rng(3)
    q = rng.standard_normal((T, 2, D)).astype(np.float32)
    p = rng.standard_normal((2, n_cells, D)).astype(np.float32)
    got = oracle.score(T, pos0, budget, q, p)
    for t in range(T):
        n = pos0 + t + 1
        for g in range(2):
            want = [sum(float(q[t, g, d]) * float(p[g, c, d]) for d in range(D)) for c in range(n)]
            np.testing.assert_allclose(got[t, g, :n], want, rtol=1e-13, atol=1e-13)
            assert np.isnan(got[t, g, n:]).all()


def test_score_rows_under_budget_are_not_written():
    """Rows that see at most budget cells take identity ids and need no
    scores: the oracle leaves them as they were."""
    T, pos0, budget, D = 8, 10, 14, 4   # tokens 0..3 see <= 14 cells
    q = np.ones((T, 2, D), np.float32)
    p = np.ones((2, pos0 + T, D), np.float32)
    got = oracle.score(T, pos0, budget, q, p)
    for t in range(T):
        n = pos0 + t + 1
        if n <= budget:
            assert np.isnan(got[t]).all()
        else:
            assert (got[t, :, :n] == D).all() and np.isnan(got[t, :, n:]).all()


def test_score_closed_form_of_unit_keys():
    """pooled[g][c] = (c + 1) e_{(c + g) mod D}: the score picks one element
    of the index query, scaled exactly -- a wrong cell, group or element
    index, or a transposed operand, changes it."""
    T, pos0, budget, D = 3, 70, 20, 8
    n_cells = pos0 + T
    rng = np.random.default_rng(9)
    q = rng.standard_normal((T, 2, D)).astype(np.float32)
    p = np.zeros((2, n_cells, D), np.float32)
    for g in range(2):
        for c in range(n_cells):
            p[g, c, (c + g) % D] = c + 1
    got = oracle.score(T, pos0, budget, q, p)
    for t in range(T):
        for g in range(2):
            n = pos0 + t + 1
            want = np.array([(c + 1) * float(q[t, g, (c + g) % D]) for c in range(n)])
            assert np.array_equal(got[t, g, :n], want)


def test_score_is_linear_in_the_index_query():
    T, pos0, budget, D = 4, 30, 8, 16
    rng = np.random.default_rng(11)
    q = rng.standard_normal((T, 2, D)).astype(np.float32)
    p = rng.standard_normal((2, pos0 + T, D)).astype(np.float32)
    a = oracle.score(T, pos0, budget, q, p)
    b = oracle.score(T, pos0, budget, 2 * q, p)
    ok = ~np.isnan(a)
    assert np.array_equal(b[ok], 2 * a[ok])
