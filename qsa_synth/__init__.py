"""Seeded synthetic inputs for the QSA prompt-attention path.

This module only draws random arrays; it holds none of the method's
arithmetic.  Both the fp64 oracle (``oracle/``) and the HIP path
(``quantized_sparse_flash_amd``) are fed from here, so their inputs are
identical bit for bit.

Workload shapes follow the pages:
  * 2 KV groups x 12 query heads, head dim 256 ("round 6 track b - qsa
    flash", experiment contract and delivered change; "opus_r9_qsa", what
    changed: HPG x QCH);
  * int8 K/V codes with one fp16 scale per 64 dims (a half4 per cell)
    ("round 6 track b - qsa flash", delivered change);
  * deterministic random inputs from rng seed 5 ("round 6 track b - qsa
    flash", actual runs);
  * a 2051-cell selection budget ("round 6 track b - qsa flash", delivered
    change).

The value distributions (queries N(0,1) as fp16, codes uniform in
[-127, 127], scales uniform in [0.002, 0.02], selection scores N(0,1) fp32)
are a chosen recipe: the pages name the kinds of inputs but not their
distributions.

Generator: numpy PCG64 seeded with the tuple (seed, T, pos0, layer); draws
happen in a fixed order (q, kq, ksc, vq, vsc, scores) so that adding the
optional score draw never changes the other arrays.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

N_GROUPS = 2
HEADS_PER_GROUP = 12
HEAD_DIM = 256
SCALE_BLOCK = 64
BUDGET = 2051
CHUNK = 64
SEED = 5


@dataclasses.dataclass
class LayerInputs:
    """One layer's synthetic inputs (host numpy arrays)."""

    T: int
    pos0: int
    budget: int
    n_cells: int
    q: np.ndarray            # [T][G*HPG][D] float16
    kq: np.ndarray           # [G][n_cells][D] int8
    ksc: np.ndarray          # [G][n_cells][D/64] float16
    vq: np.ndarray           # [G][n_cells][D] int8
    vsc: np.ndarray          # [G][n_cells][D/64] float16
    scores: Optional[np.ndarray]  # [T][G][n_cells] float32, or None

    @property
    def n_groups(self) -> int:
        return self.kq.shape[0]

    @property
    def heads_per_group(self) -> int:
        return self.q.shape[1] // self.kq.shape[0]

    @property
    def head_dim(self) -> int:
        return self.q.shape[2]


def layer_inputs(T: int, pos0: int, layer: int = 0, seed: int = SEED, *,
                 budget: int = BUDGET, n_cells: Optional[int] = None,
                 n_groups: int = N_GROUPS, heads_per_group: int = HEADS_PER_GROUP,
                 head_dim: int = HEAD_DIM, with_scores: Optional[bool] = None,
                 code_max: int = 127, scale_lo: float = 0.002,
                 scale_hi: float = 0.02) -> LayerInputs:
    """Draw one layer's inputs.

    ``n_cells`` defaults to ``pos0 + T`` (the KV history holds every cell a
    token of this prompt chunk can see).  Scores are drawn when some token
    is above budget (``pos0 + T > budget``) unless ``with_scores`` forces it.
    """
    if n_cells is None:
        n_cells = pos0 + T
    if n_cells < pos0 + T:
        raise ValueError("n_cells must cover pos0 + T")
    if with_scores is None:
        with_scores = pos0 + T > budget
    rng = np.random.default_rng([seed, T, pos0, layer])
    H = n_groups * heads_per_group
    nb = head_dim // SCALE_BLOCK
    q = rng.standard_normal((T, H, head_dim), dtype=np.float32).astype(np.float16)
    kq = rng.integers(-code_max, code_max + 1, (n_groups, n_cells, head_dim), dtype=np.int8)
    ksc = rng.uniform(scale_lo, scale_hi, (n_groups, n_cells, nb)).astype(np.float16)
    vq = rng.integers(-code_max, code_max + 1, (n_groups, n_cells, head_dim), dtype=np.int8)
    vsc = rng.uniform(scale_lo, scale_hi, (n_groups, n_cells, nb)).astype(np.float16)
    scores = None
    if with_scores:
        scores = rng.standard_normal((T, n_groups, n_cells), dtype=np.float32)
    return LayerInputs(T=T, pos0=pos0, budget=budget, n_cells=n_cells, q=q, kq=kq,
                       ksc=ksc, vq=vq, vsc=vsc, scores=scores)


@dataclasses.dataclass
class SparseHistory:
    """Inputs over a KV history too long to draw whole: the selected ids of
    every (token, group) row, and codes and scales for only the cells that
    some row selects.  cells[g] lists group g's selected cells (sorted,
    unique); kq[g][i] etc. belong to cell cells[g][i]."""

    T: int
    pos0: int
    budget: int
    n_cells: int
    q: np.ndarray            # [T][G*HPG][D] float16
    ids: np.ndarray          # [T][G][budget] int32, each row sorted ascending
    cells: list              # G arrays of int64
    kq: list                 # G arrays [len(cells[g])][D] int8
    ksc: list                # G arrays [len(cells[g])][D/64] float16
    vq: list
    vsc: list


def sparse_history(T: int, pos0: int, n_cells: int, seed: int = SEED, *, budget: int = BUDGET,
                   n_groups: int = N_GROUPS, heads_per_group: int = HEADS_PER_GROUP,
                   head_dim: int = HEAD_DIM, recent: int = 4096,
                   recent_share: float = 0.25) -> SparseHistory:
    """Ids and cell data for tokens that all see more than ``budget`` cells.

    Each row takes ``recent_share`` of its budget from its last ``recent``
    visible cells and the rest from the cells before them (uniform, without
    replacement), sorted ascending; codes, scales and queries follow the
    distributions of layer_inputs."""
    if pos0 + 1 <= budget + recent or n_cells < pos0 + T:
        raise ValueError("every token must see more than budget + recent cells")
    rng = np.random.default_rng([seed, T, pos0, n_cells, 41])
    H = n_groups * heads_per_group
    nb = head_dim // SCALE_BLOCK
    q = rng.standard_normal((T, H, head_dim), dtype=np.float32).astype(np.float16)
    ids = np.empty((T, n_groups, budget), dtype=np.int32)
    n_recent = int(budget * recent_share)
    for t in range(T):
        nkv = pos0 + t + 1
        for g in range(n_groups):
            old = rng.choice(nkv - recent, budget - n_recent, replace=False)
            new = nkv - recent + rng.choice(recent, n_recent, replace=False)
            ids[t, g] = np.sort(np.concatenate([old, new]))
    cells, kq, ksc, vq, vsc = [], [], [], [], []
    for g in range(n_groups):
        c = np.unique(ids[:, g, :]).astype(np.int64)
        cells.append(c)
        kq.append(rng.integers(-127, 128, (len(c), head_dim), dtype=np.int8))
        ksc.append(rng.uniform(0.002, 0.02, (len(c), nb)).astype(np.float16))
        vq.append(rng.integers(-127, 128, (len(c), head_dim), dtype=np.int8))
        vsc.append(rng.uniform(0.002, 0.02, (len(c), nb)).astype(np.float16))
    return SparseHistory(T=T, pos0=pos0, budget=budget, n_cells=n_cells, q=q, ids=ids,
                         cells=cells, kq=kq, ksc=ksc, vq=vq, vsc=vsc)


def score_inputs(T: int, pos0: int, index_dim: int = 4, seed: int = SEED, *,
                 n_groups: int = N_GROUPS, n_cells: Optional[int] = None) -> tuple:
    """Inputs of the selection-score step: qidx [T][G][index_dim] and pooled
    [G][n_cells][index_dim], both N(0,1) fp32 (a chosen recipe; the pages
    name the buffers, not their distributions)."""
    if n_cells is None:
        n_cells = pos0 + T
    rng = np.random.default_rng([seed, T, pos0, index_dim, 43])
    qidx = rng.standard_normal((T, n_groups, index_dim), dtype=np.float32)
    pooled = rng.standard_normal((n_groups, n_cells, index_dim), dtype=np.float32)
    return qidx, pooled


def score_rows(T: int, n_groups: int, n_cells: int, seed: int, *, kind: str = "normal",
               levels: int = 4) -> np.ndarray:
    """Selection-score arrays for top-k tests.

    kind:
      "normal"    N(0,1) fp32 (the workload's scores);
      "quantized" N(0,1) rounded to ``levels`` distinct values (many ties);
      "signed_zero"  a mix of +0.0, -0.0 and a few N(0,1) values.
    """
    rng = np.random.default_rng([seed, T, n_cells, 17])
    s = rng.standard_normal((T, n_groups, n_cells), dtype=np.float32)
    if kind == "normal":
        return s
    if kind == "quantized":
        return np.floor(s * (levels / 4.0)).astype(np.float32)
    if kind == "signed_zero":
        sign = rng.integers(0, 2, s.shape).astype(bool)
        z = np.where(sign, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
        keep = rng.random(s.shape) < 0.05
        return np.where(keep, s, z).astype(np.float32)
    raise ValueError(kind)


def kv_rows(n_rows: int, seed: int = SEED, *, kind: str = "mixed") -> np.ndarray:
    """Unquantised fp16 K/V rows [n_rows][256] for quantiser tests and the
    quantiser workload.

    kind:
      "mixed"  N(0,1) times a per-(row, 64-dim block) magnitude 10^U(-3, 1),
               so blocks span tiny to large values (pre-quantisation K/V);
      "edge"   blocks that are all zero, a single +-fp16 subnormal, the
               fp16 extremes (+-65504), exact halves of the scale, or mixed.
    """
    rng = np.random.default_rng([seed, n_rows, 29])
    if kind == "mixed":
        mag = np.power(10.0, rng.uniform(-3.0, 1.0, (n_rows, HEAD_DIM // SCALE_BLOCK, 1)))
        x = rng.standard_normal((n_rows, HEAD_DIM // SCALE_BLOCK, SCALE_BLOCK)) * mag
        return x.reshape(n_rows, HEAD_DIM).astype(np.float16)
    if kind == "edge":
        nb = HEAD_DIM // SCALE_BLOCK
        x = np.zeros((n_rows, nb, SCALE_BLOCK))
        pick = rng.integers(0, 5, (n_rows, nb))
        for r in range(n_rows):
            for b in range(nb):
                p = pick[r, b]
                if p == 1:
                    x[r, b, rng.integers(SCALE_BLOCK)] = rng.choice([-1, 1]) * 2.0 ** -24
                elif p == 2:
                    x[r, b] = rng.choice([-65504.0, 65504.0, 1.0, -3.0], SCALE_BLOCK)
                elif p == 3:
                    x[r, b] = rng.integers(-126, 126, SCALE_BLOCK) + 0.5
                    x[r, b, 0] = 127.0
                elif p == 4:
                    x[r, b] = rng.standard_normal(SCALE_BLOCK) * 10.0 ** rng.uniform(-8, 4)
        return np.clip(x, -65504.0, 65504.0).reshape(n_rows, HEAD_DIM).astype(np.float16)
    raise ValueError(kind)


# Named workloads (sizes of the pages' measured configurations).
WORKLOADS = {
    # tiny prompt under budget: token t sees cells 0..t; one layer
    "t96_pos0": dict(T=96, pos0=0, layers=1),
    # 12 back-to-back layers at pos0 0 (identity selection)
    "t512_pos0_x12": dict(T=512, pos0=0, layers=12),
    "t1024_pos0_x12": dict(T=1024, pos0=0, layers=12),
    "t1984_pos0_x12": dict(T=1984, pos0=0, layers=12),
    # chunks that cross the 2051-cell budget
    "t96_pos2050": dict(T=96, pos0=2050, layers=1),
    "t32_pos2050": dict(T=32, pos0=2050, layers=1),
    # long context: every token takes its top-2051 of ~32K cells
    "t1984_pos30000": dict(T=1984, pos0=30000, layers=1),
    # decode-merge: 4 tokens at position 8192, split into 64-cell chunks
    "decode4_pos8192": dict(T=4, pos0=8192, layers=1),
}
