"""GPU parity of qsa_quantize against the oracle's K/V quantiser.

Codes and scales are integers decided in IEEE fp32 on both sides, so the
bar is bit-exactness.  The end-to-end case quantises fp16 K/V on the GPU and
feeds the codes to qsa_flash, against the oracle run on the oracle's own
quantisation of the same rows.
"""
import numpy as np
import pytest
import torch

import oracle
import qsa_synth
import quantized_sparse_flash_amd as qsa
from gpu_util import DEV, gpu_flash

pytestmark = pytest.mark.gpu


def _gpu_quantize(x: np.ndarray):
    xt = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    codes = torch.full(x.shape, 99, dtype=torch.int8, device=DEV)
    scales = torch.full(x.shape[:-1] + (4,), float("nan"), dtype=torch.float16, device=DEV)
    qsa.qsa_quantize(xt, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def _assert_same(x):
    c, s = _gpu_quantize(x)
    rc, rs = oracle.quantize(x)
    assert np.array_equal(s.view(np.uint16), rs.view(np.uint16))
    bad = np.argwhere(c != rc)
    assert bad.size == 0, "first mismatch at %s: gpu %d oracle %d" % (
        bad[0], c[tuple(bad[0])], rc[tuple(bad[0])])


@pytest.mark.parametrize("rows", [1, 3, 16, 17, 1000])
def test_quantize_matches_oracle_mixed(rows):
    _assert_same(qsa_synth.kv_rows(rows, kind="mixed"))


@pytest.mark.parametrize("rows", [5, 33, 400])
def test_quantize_matches_oracle_edge_blocks(rows):
    _assert_same(qsa_synth.kv_rows(rows, kind="edge"))


def test_quantize_long_context_cache_full_size():
    # the K history of the long-context workload: 2 groups x 31,984 cells
    x = qsa_synth.kv_rows(2 * 31984, seed=3).reshape(2, 31984, 256)
    _assert_same(x)


def test_quantize_then_flash_end_to_end():
    T, pos0 = 96, 0
    base = qsa_synth.layer_inputs(T, pos0, seed=5)
    n = base.n_cells
    k16 = qsa_synth.kv_rows(2 * n, seed=6).reshape(2, n, 256)
    v16 = qsa_synth.kv_rows(2 * n, seed=7).reshape(2, n, 256)
    kq, ksc = _gpu_quantize(k16)
    vq, vsc = _gpu_quantize(v16)
    okq, oksc = oracle.quantize(k16)
    ovq, ovsc = oracle.quantize(v16)
    assert np.array_equal(kq, okq) and np.array_equal(vq, ovq)
    inp = qsa_synth.LayerInputs(T=T, pos0=pos0, budget=base.budget, n_cells=n, q=base.q,
                                kq=kq, ksc=ksc, vq=vq, vsc=vsc, scores=None)
    ref = oracle.attend(qsa_synth.LayerInputs(T=T, pos0=pos0, budget=base.budget, n_cells=n,
                                              q=base.q, kq=okq, ksc=oksc, vq=ovq, vsc=ovsc,
                                              scores=None), None)
    got = gpu_flash(inp)
    assert np.all(np.isfinite(got))
    assert oracle.rel_l2(got, ref) <= 1e-3


def test_quantize_zero_rows_is_a_no_op():
    x = torch.zeros((0, 256), dtype=torch.float16, device=DEV)
    c = torch.zeros((0, 256), dtype=torch.int8, device=DEV)
    s = torch.zeros((0, 4), dtype=torch.float16, device=DEV)
    qsa.qsa_quantize(x, c, s)
    torch.cuda.synchronize()
