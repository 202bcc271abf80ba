"""fp64 CPU oracle for the QSA prompt-attention path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  It
shares no code with the HIP library (``quantized_sparse_flash_amd``) and
never imports it; the two meet only in the seeded input generator
``qsa_synth``, which holds no arithmetic of the method.

Two independent formulations live here:
  * ``qsa_oracle.c`` (built with gcc, OpenMP over (token, group) rows): the
    plain definition -- selection, then exact softmax attention over the
    selected cells -- plus the selection scores (the reading of the
    score kernel: an fp64 dot product of index query and pooled key), the
    chunk-partial and log-sum-exp merge steps, and the K/V quantiser that
    fills the int8 cache (decided in IEEE fp32);
  * ``dense_reference`` below: a numpy brute force over the full (token x
    cell) matrix with explicit causal and top-k masks, for tiny inputs.

Pinning (tests/test_oracle_pins.py): the C oracle is checked against the
brute force, against torch's scaled_dot_product_attention (CPU, fp64) where
selection is the identity, against numpy's stable argsort for selection,
against closed forms (one visible cell, zero key scales) and against the
split/merge and scaling invariants.  Parity is pinned for every function
here; nothing is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qsa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libqsa_oracle.so")
# Set only by tests/test_oracle_mutants.py, in the child processes it starts:
# a build of qsa_oracle.c with one planted mistake, which the pins must reject.
_MUTANT_ENV = "QSA_ORACLE_MUTANT_LIB"
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (OpenMP).  Returns the library path."""
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get(_MUTANT_ENV)
    if not path:
        path = _LIB_PATH
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
            build(force=True)
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    lib.qsa_oracle_select.argtypes = [i32, i32, i32, i32, i64, P, P]
    lib.qsa_oracle_score.argtypes = [i32, i32, i32, i32, i32, i64, P, P, P]
    lib.qsa_oracle_attend.argtypes = [i32, i32, i32, i32, i32, i32, i64, P, P, P, P, P, P, P]
    lib.qsa_oracle_partials.argtypes = [i32, i32, i32, i32, i32, i32, i64, i32,
                                        P, P, P, P, P, P, P, P, P]
    lib.qsa_oracle_merge.argtypes = [i32, i32, i32, i32, P, P, P]
    lib.qsa_oracle_quantize.argtypes = [i64, i32, i32, P, P, P]
    lib.qsa_oracle_f32_to_f16.argtypes = [i64, P, P]
    for f in (lib.qsa_oracle_select, lib.qsa_oracle_score, lib.qsa_oracle_attend, lib.qsa_oracle_partials,
              lib.qsa_oracle_merge, lib.qsa_oracle_quantize, lib.qsa_oracle_f32_to_f16):
        f.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def n_selected(pos0: int, t: int, budget: int) -> int:
    """Cells token t attends: all pos0+t+1 visible cells, capped at budget."""
    return min(pos0 + t + 1, budget)


def score(T: int, pos0: int, budget: int, qidx: np.ndarray, pooled: np.ndarray) -> np.ndarray:
    """Selection scores [T][G][n_cells] (fp64) of the rows above budget at
    their visible cells; NaN everywhere else.  qidx [T][G][D], pooled
    [G][n_cells][D]."""
    lib = _load()
    G, n_cells, D = pooled.shape
    if qidx.shape != (T, G, D):
        raise ValueError("qidx shape")
    out = np.full((T, G, n_cells), np.nan, dtype=np.float64)
    rc = lib.qsa_oracle_score(T, pos0, G, D, budget, n_cells, _ptr(_c(qidx, np.float64)),
                              _ptr(_c(pooled, np.float64)), _ptr(out))
    if rc != 0:
        raise RuntimeError("qsa_oracle_score failed")
    return out


def select(T: int, pos0: int, budget: int, scores: Optional[np.ndarray], n_groups: int,
           n_cells: int) -> np.ndarray:
    """ids[T][G][budget] int32 (identity rows 0..n-1 then -1)."""
    lib = _load()
    ids = np.empty((T, n_groups, budget), dtype=np.int32)
    sc = None if scores is None else _c(scores, np.float32)
    if sc is not None and sc.shape != (T, n_groups, n_cells):
        raise ValueError("scores shape")
    rc = lib.qsa_oracle_select(T, pos0, n_groups, budget, n_cells, _ptr(sc), _ptr(ids))
    if rc != 0:
        raise RuntimeError("qsa_oracle_select failed")
    return ids


def attend(inp, ids: Optional[np.ndarray]) -> np.ndarray:
    """Full fp64 output [T][H][D] for LayerInputs ``inp`` and selected ids."""
    lib = _load()
    T, H, D = inp.q.shape
    G = inp.kq.shape[0]
    q = _c(inp.q, np.float64)
    ksc = _c(inp.ksc, np.float64)
    vsc = _c(inp.vsc, np.float64)
    kq = _c(inp.kq, np.int8)
    vq = _c(inp.vq, np.int8)
    idc = None if ids is None else _c(ids, np.int32)
    out = np.empty((T, H, D), dtype=np.float64)
    rc = lib.qsa_oracle_attend(T, inp.pos0, G, H // G, D, inp.budget, inp.n_cells, _ptr(q),
                               _ptr(kq), _ptr(ksc), _ptr(vq), _ptr(vsc), _ptr(idc), _ptr(out))
    if rc != 0:
        raise RuntimeError("qsa_oracle_attend failed")
    return out


def partials(inp, ids: Optional[np.ndarray], chunk: int = 64):
    """Chunk partials (m, l, o): m, l [T][KC][H]; o [T][KC][H][D]; KC =
    ceil(budget / chunk).  Entries of chunks a token lacks are NaN."""
    lib = _load()
    T, H, D = inp.q.shape
    G = inp.kq.shape[0]
    KC = -(-inp.budget // chunk)
    m = np.full((T, KC, H), np.nan)
    l = np.full((T, KC, H), np.nan)
    o = np.full((T, KC, H, D), np.nan)
    idc = None if ids is None else _c(ids, np.int32)
    rc = lib.qsa_oracle_partials(T, inp.pos0, G, H // G, D, inp.budget, inp.n_cells, chunk,
                                 _ptr(_c(inp.q, np.float64)), _ptr(_c(inp.kq, np.int8)),
                                 _ptr(_c(inp.ksc, np.float64)), _ptr(_c(inp.vq, np.int8)),
                                 _ptr(_c(inp.vsc, np.float64)), _ptr(idc), _ptr(m), _ptr(l),
                                 _ptr(o))
    if rc != 0:
        raise RuntimeError("qsa_oracle_partials failed")
    return m, l, o


def chunk_counts(T: int, pos0: int, budget: int, chunk: int = 64) -> np.ndarray:
    """Chunks per token of the split form: ceil(n_sel(t) / chunk)."""
    return np.array([-(-n_selected(pos0, t, budget) // chunk) for t in range(T)], dtype=np.int32)


def pack_part(m, l, o) -> np.ndarray:
    """fp32 record layout [T][KC][H][D+2] = (o, m, l) of the split form.
    Missing chunks (NaN in the oracle arrays) are packed as zeros."""
    T, KC, H, D = o.shape
    part = np.zeros((T, KC, H, D + 2), dtype=np.float32)
    ok = np.isfinite(m)
    part[..., :D] = np.where(ok[..., None], o, 0.0)
    part[..., D] = np.where(ok, m, 0.0)
    part[..., D + 1] = np.where(ok, l, 0.0)
    return part


def merge(part: np.ndarray, nchunks: np.ndarray) -> np.ndarray:
    """fp64 log-sum-exp merge of fp32 records [T][KC][H][D+2]."""
    lib = _load()
    T, KC, H, R = part.shape
    D = R - 2
    out = np.empty((T, H, D), dtype=np.float64)
    rc = lib.qsa_oracle_merge(T, H, D, KC, _ptr(_c(nchunks, np.int32)),
                              _ptr(_c(part, np.float32)), _ptr(out))
    if rc != 0:
        raise RuntimeError("qsa_oracle_merge failed")
    return out


def dense_reference(inp, scores: Optional[np.ndarray] = None) -> tuple:
    """Brute force over the whole (token x cell) matrix, for tiny inputs.

    Builds the dequantised K, V, the full fp64 score matrix for every head,
    a boolean mask per (t, g) -- causal visibility, then the top-``budget``
    cells by a rank count when the token is above budget -- and applies a
    masked softmax.  Returns (out [T][H][D], mask [T][G][N]).
    Written independently of qsa_oracle.c: no chunking, no per-row lists.
    """
    T, H, D = inp.q.shape
    G, N, _ = inp.kq.shape
    HPG = H // G
    B = inp.budget
    k = inp.kq.astype(np.float64) * np.repeat(inp.ksc.astype(np.float64), 64, axis=2)
    v = inp.vq.astype(np.float64) * np.repeat(inp.vsc.astype(np.float64), 64, axis=2)
    q = inp.q.astype(np.float64)
    pos = inp.pos0 + np.arange(T)
    visible = np.arange(N)[None, :] <= pos[:, None]          # [T][N]
    mask = np.zeros((T, G, N), dtype=bool)
    for t in range(T):
        for g in range(G):
            vis = visible[t]
            if vis.sum() <= B:
                mask[t, g] = vis
                continue
            s = scores[t, g].astype(np.float64)
            # rank = #{strictly greater} + #{equal with lower index}, over
            # visible cells only; selected iff rank < B
            for c in np.nonzero(vis)[0]:
                greater = np.sum(vis & (s > s[c]))
                tie_before = np.sum(vis[:c] & (s[:c] == s[c]))
                mask[t, g, c] = (greater + tie_before) < B
    out = np.empty((T, H, D))
    for h in range(H):
        g = h // HPG
        logits = (q[:, h, :] @ k[g].T) / np.sqrt(D)          # [T][N]
        logits = np.where(mask[:, g, :], logits, -np.inf)
        mx = logits.max(axis=1, keepdims=True)
        w = np.exp(logits - mx)
        w /= w.sum(axis=1, keepdims=True)
        out[:, h, :] = w @ v[g]
    return out, mask


def f32_to_f16(a: np.ndarray) -> np.ndarray:
    """The oracle's own fp32 -> fp16 rounding (to nearest, ties to even)."""
    lib = _load()
    x = _c(a, np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    if lib.qsa_oracle_f32_to_f16(x.size, _ptr(x), _ptr(out)) != 0:
        raise RuntimeError("qsa_oracle_f32_to_f16 failed")
    return out.view(np.float16)


def quantize(x: np.ndarray, block: int = 64) -> tuple:
    """K/V quantiser: fp16 rows [..., D] -> (int8 codes [..., D], fp16
    scales [..., D / block]); per block scale = fp16(absmax / 127) and
    code = clamp(rint(x / scale), -127, 127), decided in IEEE fp32."""
    lib = _load()
    xh = np.ascontiguousarray(x, dtype=np.float16)
    D = xh.shape[-1]
    rows = xh.size // D if D else 0
    codes = np.empty(xh.shape, dtype=np.int8)
    scales = np.empty(xh.shape[:-1] + (D // block,), dtype=np.uint16)
    rc = lib.qsa_oracle_quantize(rows, D, block, _ptr(xh.view(np.uint16)), _ptr(codes),
                                 _ptr(scales))
    if rc != 0:
        raise RuntimeError("qsa_oracle_quantize failed")
    return codes, scales.view(np.float16)


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    """||a - b||_2 / ||b||_2 over the whole tensor (b is the reference)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-300))
