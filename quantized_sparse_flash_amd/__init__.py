"""quantized_sparse_flash_amd -- the QSA prompt-attention path on MI355X.

A thin ctypes binding over ``libqsa.so`` (C ABI in ``include/qsa.h``).  The
functions carry the C names and only marshal arguments: shapes, dtypes and
devices are checked, device pointers and the current HIP stream are passed
through, and every step of the path runs in the library's gfx950 kernels.
PyTorch supplies device memory and streams.  There is no CPU fallback: if
the library is missing or cannot be loaded, calls raise.

Entry points (all asynchronous on the current stream):
  qsa_topk(shape, scores, ids)                                 selection
  qsa_flash(shape, q, kq, ksc, vq, vsc, ids, out, part=None)   attention
  qsa_flash_prepare(shape, kq, ksc, vq, vsc, workspace)         fused mode, first half
  qsa_flash_attend(shape, q, kq, ksc, vq, vsc, ids, out, workspace)   ... second half
  qsa_flash_noalloc(shape, q, kq, ksc, vq, vsc, ids, out, part=None)
                                                    qsa_flash with library-held scratch
  qsa_merge(shape, part, out)                                  LSE merge
  qsa_quantize(x, codes, scales)                               K/V quantiser
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libqsa.so")

QSA_OK = 0
QSA_ERR_ARG = -1
QSA_ERR_UNSUPPORTED = -2
QSA_ERR_SHAPE = -3
QSA_ERR_LAUNCH = -4
QSA_ERR_TOO_LARGE = -5
QSA_ERR_DEVICE = -6
NOALLOC_SCRATCH_BYTES = 16 << 20
HEADS_PER_GROUP = 12
HEAD_DIM = 256
CHUNK = 64
PART_STRIDE = 258
DEFAULT_BUDGET = 2051
MAX_BUDGET = 65536
MAX_INDEX_DIM = 256  # longest qsa_score vectors

EXPORTED = ("qsa_score", "qsa_topk", "qsa_flash", "qsa_flash_prepare", "qsa_flash_attend",
            "qsa_merge", "qsa_quantize", "qsa_status_string", "qsa_part_elems",
            "qsa_flash_workspace_bytes", "qsa_flash_noalloc")


class QsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__("%s: %s (status %d)" % (where, qsa_status_string(status), status))
        self.status = status


class _CShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("pos0", ctypes.c_int32), ("n_groups", ctypes.c_int32),
                ("heads_per_group", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("budget", ctypes.c_int32), ("n_cells", ctypes.c_int64)]


@dataclasses.dataclass
class QsaShape:
    """Mirror of the C ``qsa_shape``; ``n_cells`` defaults to pos0 + T."""

    T: int
    pos0: int
    n_groups: int = 2
    budget: int = DEFAULT_BUDGET
    n_cells: Optional[int] = None
    heads_per_group: int = HEADS_PER_GROUP
    head_dim: int = HEAD_DIM

    def __post_init__(self):
        if self.n_cells is None:
            self.n_cells = self.pos0 + self.T

    @property
    def n_heads(self) -> int:
        return self.n_groups * self.heads_per_group

    @property
    def n_part_chunks(self) -> int:
        return -(-self.budget // CHUNK)

    def c(self) -> _CShape:
        return _CShape(self.T, self.pos0, self.n_groups, self.heads_per_group, self.head_dim,
                       self.budget, self.n_cells)


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libqsa.so (raises if it is absent: build it with
    ``python -m quantized_sparse_flash_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libqsa.so not built (%s); run `python -m "
                           "quantized_sparse_flash_amd.build`" % path)
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    SP = ctypes.POINTER(_CShape)
    lib.qsa_score.argtypes = [SP, ctypes.c_int32, P, P, P, P]
    lib.qsa_topk.argtypes = [SP, P, P, P]
    lib.qsa_flash.argtypes = [SP, P, P, P, P, P, P, P, P, P, ctypes.c_int64, P]
    lib.qsa_flash_prepare.argtypes = [SP, P, P, P, P, P, ctypes.c_int64, P]
    lib.qsa_flash_attend.argtypes = [SP, P, P, P, P, P, P, P, P, ctypes.c_int64, P]
    lib.qsa_flash_noalloc.argtypes = [SP, P, P, P, P, P, P, P, P, P]
    lib.qsa_flash_workspace_bytes.argtypes = [SP]
    lib.qsa_flash_workspace_bytes.restype = ctypes.c_int64
    lib.qsa_merge.argtypes = [SP, P, P, P]
    lib.qsa_quantize.argtypes = [ctypes.c_int64, ctypes.c_int32, P, P, P, P]
    lib.qsa_status_string.argtypes = [ctypes.c_int]
    lib.qsa_status_string.restype = ctypes.c_char_p
    lib.qsa_part_elems.argtypes = [SP]
    lib.qsa_part_elems.restype = ctypes.c_int64
    for f in (lib.qsa_score, lib.qsa_topk, lib.qsa_flash, lib.qsa_flash_prepare,
              lib.qsa_flash_attend, lib.qsa_merge, lib.qsa_quantize, lib.qsa_flash_noalloc):
        f.restype = ctypes.c_int
    _lib = lib
    return lib


def qsa_status_string(status: int) -> str:
    return load_library().qsa_status_string(int(status)).decode()


def qsa_part_elems(shape: QsaShape) -> int:
    cs = shape.c()
    return int(load_library().qsa_part_elems(ctypes.byref(cs)))


def qsa_flash_workspace_bytes(shape: QsaShape) -> int:
    cs = shape.c()
    return int(load_library().qsa_flash_workspace_bytes(ctypes.byref(cs)))


_ws_cache = {}


def flash_workspace(shape: QsaShape, device=None):
    """A uint8 device tensor large enough for qsa_flash on ``shape`` (kept
    and reused per device; grows when a larger one is needed), or None."""
    import torch
    need = qsa_flash_workspace_bytes(shape)
    if need == 0:
        return None
    dev = torch.device(device if device is not None else "cuda")
    key = (dev.type, dev.index if dev.index is not None else torch.cuda.current_device())
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        _ws_cache[key] = ws
    return ws


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev_ptr(t, name, dtype, shape=None):
    """Device pointer of a contiguous CUDA tensor of the given dtype/shape."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    return ctypes.c_void_p(t.data_ptr())


def _score_args(s: QsaShape, qidx, pooled, scores) -> list:
    import torch
    if qidx is None or qidx.dim() != 3:
        raise ValueError("qidx must be a [T][G][index_dim] float32 device tensor")
    dim = int(qidx.shape[2])
    return [ctypes.c_int32(dim),
            _dev_ptr(qidx, "qidx", torch.float32, (s.T, s.n_groups, dim)),
            _dev_ptr(pooled, "pooled", torch.float32, (s.n_groups, s.n_cells, dim)),
            _dev_ptr(scores, "scores", torch.float32, (s.T, s.n_groups, s.n_cells))]


def qsa_score(shape: QsaShape, qidx, pooled, scores, stream=None) -> None:
    """Selection scores of the rows above budget: scores[t][g][c] =
    qidx[t][g] . pooled[g][c] (fp32) for c < n_kv(t); index_dim is
    qidx.shape[2]."""
    s = shape
    cs = s.c()
    rc = load_library().qsa_score(ctypes.byref(cs), *_score_args(s, qidx, pooled, scores),
                                  _stream(stream))
    if rc != QSA_OK:
        raise QsaError(rc, "qsa_score")


def qsa_topk(shape: QsaShape, scores, ids, stream=None) -> None:
    """Write selected ids [T][G][budget] (int32) for every (token, group)."""
    import torch
    s = shape
    sc = _dev_ptr(scores, "scores", torch.float32, (s.T, s.n_groups, s.n_cells))
    ip = _dev_ptr(ids, "ids", torch.int32, (s.T, s.n_groups, s.budget))
    cs = s.c()
    rc = load_library().qsa_topk(ctypes.byref(cs), sc, ip, _stream(stream))
    if rc != QSA_OK:
        raise QsaError(rc, "qsa_topk")


def qsa_flash(shape: QsaShape, q, kq, ksc, vq, vsc, ids, out, part=None, workspace=None,
              stream=None) -> None:
    """Attention over the selected cells: fused (writes ``out``) or, with
    ``part``, split mode (writes per-chunk (o, m, l) records).  ``workspace``
    (uint8 device tensor) defaults to a cached one of the needed size; calls
    in flight on different streams at once must pass their own."""
    import torch
    s = shape
    if part is None and workspace is None:
        workspace = flash_workspace(s, q.device)
    ws_ptr = None
    ws_bytes = 0
    if workspace is not None:
        ws_ptr = _dev_ptr(workspace, "workspace", torch.uint8)
        ws_bytes = workspace.numel()
    H, D, N, G = s.n_heads, s.head_dim, s.n_cells, s.n_groups
    nb = D // 64
    args = [_dev_ptr(q, "q", torch.float16, (s.T, H, D)),
            _dev_ptr(kq, "kq", torch.int8, (G, N, D)),
            _dev_ptr(ksc, "ksc", torch.float16, (G, N, nb)),
            _dev_ptr(vq, "vq", torch.int8, (G, N, D)),
            _dev_ptr(vsc, "vsc", torch.float16, (G, N, nb)),
            _dev_ptr(ids, "ids", torch.int32, (s.T, G, s.budget)),
            _dev_ptr(out, "out", torch.float16, (s.T, H, D)),
            _dev_ptr(part, "part", torch.float32, (s.T, s.n_part_chunks, H, PART_STRIDE))]
    cs = s.c()
    rc = load_library().qsa_flash(ctypes.byref(cs), *args, ws_ptr, ws_bytes, _stream(stream))
    if rc != QSA_OK:
        raise QsaError(rc, "qsa_flash")


def qsa_flash_noalloc(shape: QsaShape, q, kq, ksc, vq, vsc, ids, out, part=None,
                      stream=None) -> None:
    """qsa_flash without a workspace: the library's own static device scratch
    (NOALLOC_SCRATCH_BYTES per GPU) serves the fused path; calls that overlap
    in time on one GPU race.  Raises QsaError (QSA_ERR_TOO_LARGE) for shapes
    whose workspace would exceed that scratch."""
    import torch
    s = shape
    H, D, N, G = s.n_heads, s.head_dim, s.n_cells, s.n_groups
    args = [_dev_ptr(q, "q", torch.float16, (s.T, H, D)),
            _dev_ptr(kq, "kq", torch.int8, (G, N, D)),
            _dev_ptr(ksc, "ksc", torch.float16, (G, N, D // 64)),
            _dev_ptr(vq, "vq", torch.int8, (G, N, D)),
            _dev_ptr(vsc, "vsc", torch.float16, (G, N, D // 64)),
            _dev_ptr(ids, "ids", torch.int32, (s.T, G, s.budget)),
            _dev_ptr(out, "out", torch.float16, (s.T, H, D)),
            _dev_ptr(part, "part", torch.float32, (s.T, s.n_part_chunks, H, PART_STRIDE))]
    cs = s.c()
    rc = load_library().qsa_flash_noalloc(ctypes.byref(cs), *args, _stream(stream))
    if rc != QSA_OK:
        raise QsaError(rc, "qsa_flash_noalloc")


def _kv_args(s: QsaShape, kq, ksc, vq, vsc) -> list:
    import torch
    G, N, D = s.n_groups, s.n_cells, s.head_dim
    return [_dev_ptr(kq, "kq", torch.int8, (G, N, D)),
            _dev_ptr(ksc, "ksc", torch.float16, (G, N, D // 64)),
            _dev_ptr(vq, "vq", torch.int8, (G, N, D)),
            _dev_ptr(vsc, "vsc", torch.float16, (G, N, D // 64))]


def _ws_args(s: QsaShape, workspace, device) -> list:
    import torch
    if workspace is None:
        workspace = flash_workspace(s, device)
    if workspace is None:
        return [None, 0]
    return [_dev_ptr(workspace, "workspace", torch.uint8), workspace.numel()]


def qsa_flash_prepare(shape: QsaShape, kq, ksc, vq, vsc, workspace=None, stream=None) -> None:
    """First half of a fused qsa_flash call: dequantise the cells shared by
    the tokens under budget into ``workspace`` (nothing when there are none)."""
    s = shape
    cs = s.c()
    rc = load_library().qsa_flash_prepare(ctypes.byref(cs), *_kv_args(s, kq, ksc, vq, vsc),
                                          *_ws_args(s, workspace, kq.device), _stream(stream))
    if rc != QSA_OK:
        raise QsaError(rc, "qsa_flash_prepare")


def qsa_flash_attend(shape: QsaShape, q, kq, ksc, vq, vsc, ids, out, workspace=None,
                     stream=None) -> None:
    """Second half of a fused qsa_flash call: attention of every token, from a
    workspace filled by qsa_flash_prepare (same shape and K/V) on this stream."""
    import torch
    s = shape
    H, D = s.n_heads, s.head_dim
    args = ([_dev_ptr(q, "q", torch.float16, (s.T, H, D))] + _kv_args(s, kq, ksc, vq, vsc) +
            [_dev_ptr(ids, "ids", torch.int32, (s.T, s.n_groups, s.budget)),
             _dev_ptr(out, "out", torch.float16, (s.T, H, D))])
    cs = s.c()
    rc = load_library().qsa_flash_attend(ctypes.byref(cs), *args,
                                         *_ws_args(s, workspace, q.device), _stream(stream))
    if rc != QSA_OK:
        raise QsaError(rc, "qsa_flash_attend")


def qsa_merge(shape: QsaShape, part, out, stream=None) -> None:
    """Log-sum-exp merge of split-mode records into ``out`` [T][H][D] fp16."""
    import torch
    s = shape
    H = s.n_heads
    pp = _dev_ptr(part, "part", torch.float32, (s.T, s.n_part_chunks, H, PART_STRIDE))
    op = _dev_ptr(out, "out", torch.float16, (s.T, H, s.head_dim))
    cs = s.c()
    rc = load_library().qsa_merge(ctypes.byref(cs), pp, op, _stream(stream))
    if rc != QSA_OK:
        raise QsaError(rc, "qsa_merge")


def qsa_quantize(x, codes, scales, stream=None) -> None:
    """Quantise fp16 rows [..., 256] into int8 ``codes`` (same shape) and fp16
    ``scales`` [..., 4]: scale = fp16(absmax / 127) per 64-dim block, code =
    clamp(rint(x / scale), -127, 127)."""
    import torch
    if x.dim() < 1 or x.shape[-1] != HEAD_DIM:
        raise ValueError("x must have a last dimension of %d" % HEAD_DIM)
    rows = x.numel() // HEAD_DIM
    xp = _dev_ptr(x, "x", torch.float16)
    cp = _dev_ptr(codes, "codes", torch.int8, tuple(x.shape))
    sp = _dev_ptr(scales, "scales", torch.float16, tuple(x.shape[:-1]) + (HEAD_DIM // 64,))
    rc = load_library().qsa_quantize(rows, HEAD_DIM, xp, cp, sp, _stream(stream))
    if rc != QSA_OK:
        raise QsaError(rc, "qsa_quantize")


class BoundCall:
    """One C-ABI call with its arguments marshalled and checked once: calling
    the object enqueues the call again on the stream it was bound to.  For
    loops that issue the same launch many times (12 layers per step); the
    tensors must stay alive and in place while the object is used."""

    def __init__(self, fn, name, args, keep):
        self._fn, self._name, self._args, self._keep = fn, name, args, keep

    def __call__(self) -> None:
        rc = self._fn(*self._args)
        if rc != QSA_OK:
            raise QsaError(rc, self._name)


def bind_qsa_flash(shape: QsaShape, q, kq, ksc, vq, vsc, ids, out, part=None, workspace=None,
                   stream=None) -> BoundCall:
    """qsa_flash with the arguments of ``qsa_flash`` (checked here, once)."""
    import torch
    s = shape
    if part is None and workspace is None:
        workspace = flash_workspace(s, q.device)
    H, D, N, G = s.n_heads, s.head_dim, s.n_cells, s.n_groups
    cs = s.c()
    args = [ctypes.byref(cs),
            _dev_ptr(q, "q", torch.float16, (s.T, H, D)),
            _dev_ptr(kq, "kq", torch.int8, (G, N, D)),
            _dev_ptr(ksc, "ksc", torch.float16, (G, N, D // 64)),
            _dev_ptr(vq, "vq", torch.int8, (G, N, D)),
            _dev_ptr(vsc, "vsc", torch.float16, (G, N, D // 64)),
            _dev_ptr(ids, "ids", torch.int32, (s.T, G, s.budget)),
            _dev_ptr(out, "out", torch.float16, (s.T, H, D)),
            _dev_ptr(part, "part", torch.float32, (s.T, s.n_part_chunks, H, PART_STRIDE)),
            None if workspace is None else _dev_ptr(workspace, "workspace", torch.uint8),
            ctypes.c_int64(0 if workspace is None else workspace.numel()),
            _stream(stream)]
    return BoundCall(load_library().qsa_flash, "qsa_flash", args,
                     (cs, q, kq, ksc, vq, vsc, ids, out, part, workspace))


def bind_qsa_score(shape: QsaShape, qidx, pooled, scores, stream=None) -> BoundCall:
    """qsa_score with the arguments of ``qsa_score`` (checked here, once)."""
    s = shape
    cs = s.c()
    args = [ctypes.byref(cs)] + _score_args(s, qidx, pooled, scores) + [_stream(stream)]
    return BoundCall(load_library().qsa_score, "qsa_score", args, (cs, qidx, pooled, scores))


def bind_qsa_topk(shape: QsaShape, scores, ids, stream=None) -> BoundCall:
    """qsa_topk with the arguments of ``qsa_topk`` (checked here, once)."""
    import torch
    s = shape
    cs = s.c()
    args = [ctypes.byref(cs),
            _dev_ptr(scores, "scores", torch.float32, (s.T, s.n_groups, s.n_cells)),
            _dev_ptr(ids, "ids", torch.int32, (s.T, s.n_groups, s.budget)),
            _stream(stream)]
    return BoundCall(load_library().qsa_topk, "qsa_topk", args, (cs, scores, ids))


def bind_qsa_merge(shape: QsaShape, part, out, stream=None) -> BoundCall:
    """qsa_merge with the arguments of ``qsa_merge`` (checked here, once)."""
    import torch
    s = shape
    cs = s.c()
    args = [ctypes.byref(cs),
            _dev_ptr(part, "part", torch.float32, (s.T, s.n_part_chunks, s.n_heads, PART_STRIDE)),
            _dev_ptr(out, "out", torch.float16, (s.T, s.n_heads, s.head_dim)),
            _stream(stream)]
    return BoundCall(load_library().qsa_merge, "qsa_merge", args, (cs, part, out))
