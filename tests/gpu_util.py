"""Helpers for the GPU parity tests: upload seeded inputs, call the HIP path
through its C-ABI binding, fetch results.  No arithmetic of the method.

Every buffer the library writes (ids, out, part) is allocated inside a
larger one whose leading and trailing guard regions hold a known bit
pattern; after each call the guards must still hold it, so a write past
either end of an output fails the test that caused it."""
from __future__ import annotations

import numpy as np
import torch

import quantized_sparse_flash_amd as qsa

DEV = "cuda:0"
GUARD_BYTES = 4096  # per side; keeps the 16-byte alignment the library needs

# guard bit patterns (a NaN payload for float buffers, so that a stray read
# of a guard into a result would also show)
_GUARD_BITS = {torch.float16: 0x7E5A, torch.float32: 0x7FC0A5A5, torch.int32: -0x5A5A5A5B}
_INT_VIEW = {torch.float16: torch.int16, torch.float32: torch.int32, torch.int32: torch.int32}


class Guarded:
    """A device tensor of `shape`/`dtype` with guard regions on both sides."""

    def __init__(self, shape, dtype, fill=None):
        n = int(np.prod(shape))
        esz = torch.empty((), dtype=dtype).element_size()
        self.g = GUARD_BYTES // esz
        self.buf = torch.empty(n + 2 * self.g, dtype=dtype, device=DEV)
        self.buf.view(_INT_VIEW[dtype]).fill_(_GUARD_BITS[dtype])
        self.t = self.buf[self.g:self.g + n].view(shape)
        if fill is not None:
            self.t.fill_(fill)

    def check(self, what=""):
        bits = self.buf.view(_INT_VIEW[self.buf.dtype])
        want = _GUARD_BITS[self.buf.dtype]
        head = bits[:self.g].cpu().numpy()
        tail = bits[-self.g:].cpu().numpy()
        assert np.all(head == want), "%s: a write landed before the buffer" % what
        assert np.all(tail == want), "%s: a write landed past the end of the buffer" % what

    def numpy(self, what=""):
        torch.cuda.synchronize()
        self.check(what)
        return self.t.cpu().numpy()


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
    ids = Guarded((s.T, s.n_groups, s.budget), torch.int32, fill=-7)
    qsa.qsa_topk(s, dev.get("scores"), ids.t)
    return ids.numpy("qsa_topk ids")


def gpu_flash(inp, ids=None, dev=None, split=False):
    """Fused: returns out [T][H][D] as float64.  Split: returns the fp32
    part records [T][KC][H][258] (unwritten records hold NaN)."""
    dev = dev or upload(inp)
    s = shape_of(inp)
    idt = None if ids is None else torch.from_numpy(np.ascontiguousarray(ids, np.int32)).to(DEV)
    if split:
        part = Guarded((s.T, s.n_part_chunks, s.n_heads, qsa.PART_STRIDE), torch.float32,
                       fill=float("nan"))
        qsa.qsa_flash(s, dev["q"], dev["kq"], dev["ksc"], dev["vq"], dev["vsc"], idt, None,
                      part.t)
        return part.numpy("qsa_flash part")
    out = Guarded((s.T, s.n_heads, s.head_dim), torch.float16, fill=float("nan"))
    qsa.qsa_flash(s, dev["q"], dev["kq"], dev["ksc"], dev["vq"], dev["vsc"], idt, out.t)
    return out.numpy("qsa_flash out").astype(np.float64)


def gpu_merge(inp, part: np.ndarray) -> np.ndarray:
    s = shape_of(inp)
    pt = torch.from_numpy(np.ascontiguousarray(part, np.float32)).to(DEV)
    out = Guarded((s.T, s.n_heads, s.head_dim), torch.float16, fill=float("nan"))
    qsa.qsa_merge(s, pt, out.t)
    return out.numpy("qsa_merge out").astype(np.float64)


def worst_row_rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    num = np.linalg.norm((got - ref).reshape(-1, ref.shape[-1]), axis=1)
    den = np.linalg.norm(ref.reshape(-1, ref.shape[-1]), axis=1)
    return float(np.max(num / np.maximum(den, 1e-300)))


def gpu_split_merge(inp, ids=None, dev=None) -> np.ndarray:
    """Split qsa_flash then qsa_merge, both on the device (the records never
    leave it); returns out [T][H][D] as float64.  Both buffers are guarded."""
    dev = dev or upload(inp)
    s = shape_of(inp)
    idt = None if ids is None else torch.from_numpy(np.ascontiguousarray(ids, np.int32)).to(DEV)
    part = Guarded((s.T, s.n_part_chunks, s.n_heads, qsa.PART_STRIDE), torch.float32,
                   fill=float("nan"))
    out = Guarded((s.T, s.n_heads, s.head_dim), torch.float16, fill=float("nan"))
    qsa.qsa_flash(s, dev["q"], dev["kq"], dev["ksc"], dev["vq"], dev["vsc"], idt, None, part.t)
    qsa.qsa_merge(s, part.t, out.t)
    torch.cuda.synchronize()
    part.check("qsa_flash part")
    got = out.numpy("qsa_merge out").astype(np.float64)
    del part
    return got
