"""Helpers for the GPU parity tests: upload seeded inputs, call the HIP path
through its C-ABI binding, fetch results.  No arithmetic of the method."""
from __future__ import annotations

import numpy as np
import torch

import quantized_sparse_flash_amd as qsa

DEV = "cuda:0"


def shape_of(inp, budget=None) -> qsa.QsaShape:
    return qsa.QsaShape(T=inp.T, pos0=inp.pos0, n_groups=inp.kq.shape[0],
                        budget=inp.budget if budget is None else budget, n_cells=inp.n_cells)


def upload(inp) -> dict:
    d = {k: torch.from_numpy(np.ascontiguousarray(getattr(inp, k))).to(DEV)
         for k in ("q", "kq", "ksc", "vq", "vsc")}
    if inp.scores is not None:
        d["scores"] = torch.from_numpy(np.ascontiguousarray(inp.scores)).to(DEV)
    return d


def gpu_topk(inp, dev=None) -> np.ndarray:
    dev = dev or upload(inp)
    s = shape_of(inp)
    ids = torch.full((s.T, s.n_groups, s.budget), -7, dtype=torch.int32, device=DEV)
    qsa.qsa_topk(s, dev.get("scores"), ids)
    torch.cuda.synchronize()
    return ids.cpu().numpy()


def gpu_flash(inp, ids=None, dev=None, split=False):
    """Fused: returns out [T][H][D] as float64.  Split: returns the fp32
    part records [T][KC][H][258] (unwritten records hold NaN)."""
    dev = dev or upload(inp)
    s = shape_of(inp)
    idt = None if ids is None else torch.from_numpy(np.ascontiguousarray(ids, np.int32)).to(DEV)
    if split:
        part = torch.full((s.T, s.n_part_chunks, s.n_heads, qsa.PART_STRIDE), float("nan"),
                          dtype=torch.float32, device=DEV)
        qsa.qsa_flash(s, dev["q"], dev["kq"], dev["ksc"], dev["vq"], dev["vsc"], idt, None, part)
        torch.cuda.synchronize()
        return part.cpu().numpy()
    out = torch.full((s.T, s.n_heads, s.head_dim), float("nan"), dtype=torch.float16, device=DEV)
    qsa.qsa_flash(s, dev["q"], dev["kq"], dev["ksc"], dev["vq"], dev["vsc"], idt, out)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def gpu_merge(inp, part: np.ndarray) -> np.ndarray:
    s = shape_of(inp)
    pt = torch.from_numpy(np.ascontiguousarray(part, np.float32)).to(DEV)
    out = torch.full((s.T, s.n_heads, s.head_dim), float("nan"), dtype=torch.float16, device=DEV)
    qsa.qsa_merge(s, pt, out)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def worst_row_rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    num = np.linalg.norm((got - ref).reshape(-1, ref.shape[-1]), axis=1)
    den = np.linalg.norm(ref.reshape(-1, ref.shape[-1]), axis=1)
    return float(np.max(num / np.maximum(den, 1e-300)))
