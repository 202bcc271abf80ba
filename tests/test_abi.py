"""The C-ABI library loads, exports what include/qsa.h declares, rejects bad
arguments before launching anything, and its constants match the pages.
No compute call is made: every call here fails validation on the host."""
import ctypes
import json
import os
import re
import subprocess

import pytest

import quantized_sparse_flash_amd as qsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsa.h")
GOLDEN = os.path.join(ROOT, "tests", "golden", "page_constants.json")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qsa_[a-z_]+)\s*\(", text)))


def _header_defines():
    text = open(HEADER).read()
    return {k: int(v) for k, v in re.findall(r"#define\s+(QSA_\w+)\s+\(?(-?\d+)\)?", text)}


def test_library_exports_every_declared_symbol():
    lib = qsa.load_library()
    declared = _declared_functions()
    assert set(declared) == set(qsa.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


def test_header_constants_match_pages_and_binding():
    d = _header_defines()
    g = json.load(open(GOLDEN))
    assert d["QSA_HEADS_PER_GROUP"] == g["heads_per_group"]["value"] == qsa.HEADS_PER_GROUP
    assert d["QSA_HEAD_DIM"] == g["head_dim"]["value"] == qsa.HEAD_DIM
    assert d["QSA_CHUNK"] == g["chunk"]["value"] == qsa.CHUNK
    assert d["QSA_DEFAULT_BUDGET"] == g["budget"]["value"] == qsa.DEFAULT_BUDGET
    assert d["QSA_PART_STRIDE"] == g["part_head_stride"]["value"] == qsa.PART_STRIDE
    assert d["QSA_HEAD_DIM"] // d["QSA_SCALE_BLOCK"] == g["scales_per_cell"]["value"]
    # chunk stride of the partial records: 24 heads x 258 floats
    n_heads = g["n_groups"]["value"] * g["heads_per_group"]["value"]
    assert n_heads * d["QSA_PART_STRIDE"] == g["part_chunk_stride"]["value"]
    for k in ("QSA_OK", "QSA_ERR_ARG", "QSA_ERR_UNSUPPORTED", "QSA_ERR_SHAPE", "QSA_ERR_LAUNCH"):
        assert getattr(qsa, k) == d[k]


def test_status_strings():
    for code in (0, -1, -2, -3, -4):
        assert qsa.qsa_status_string(code)
    assert qsa.qsa_status_string(-99) == "unknown status"


def test_flash_workspace_size():
    # fused path: 64 KB per group and 64-cell chunk of the shared prefix
    assert qsa.qsa_flash_workspace_bytes(qsa.QsaShape(T=1984, pos0=0)) == 2 * 31 * 65536
    assert qsa.qsa_flash_workspace_bytes(qsa.QsaShape(T=1024, pos0=0)) == 2 * 16 * 65536
    # a tiled grid of 64-query blocks that leaves CUs idle runs its blocks
    # of at least 12 chunks as 2 or 3 pieces; the workspace then also holds,
    # per split block, one partial slot per piece (64 x 256 floats of O, then
    # (m, l) per query) and a 4-byte arrival counter (counters rounded up to
    # 256 bytes).  T=512's blocks are at most 8 chunks: nothing is split.
    slot = (64 * 256 + 2 * 64) * 4
    assert qsa.qsa_flash_workspace_bytes(qsa.QsaShape(T=512, pos0=0)) == 2 * 8 * 65536
    # up to 512 (token, group) rows above budget run as row pieces after the
    # tiled part (rounded up to 256 bytes): each piece covers cpr of a row's
    # 33 chunks, cpr = ceil(rows x 33 / 1024) (about 1024 wavefronts), and
    # writes one record per head (24 x 258 floats per piece and token).
    # T=200 at pos0 1900 tiles its 151 tokens under budget (29 blocks of 64
    # queries per group, 33 chunks each, in 3 pieces) and splits its 49
    # tokens above (98 rows: cpr 4, 9 pieces per row)
    def rec(tokens):
        cpr = -(-tokens * 2 * 33 // 1024)
        return tokens * -(-33 // cpr) * 24 * 258 * 4
    tile = 2 * 33 * 65536 + 256 + 3 * (2 * 29) * slot
    assert rec(49) == 49 * 9 * 24 * 258 * 4
    assert qsa.qsa_flash_workspace_bytes(qsa.QsaShape(T=200, pos0=1900)) == \
        (tile + 255) // 256 * 256 + rec(49)
    # a call of at most 256 rows with some above budget splits every token
    # (the budget-crossing chunk: 192 rows, cpr 7, 5 pieces per row), and
    # with none under budget as well; up to 512 rows above budget run as
    # pieces (258 rows: cpr 9, 4 pieces per row); past 512 rows the row
    # kernel needs no workspace
    assert rec(96) == 96 * 5 * 24 * 258 * 4
    assert qsa.qsa_flash_workspace_bytes(qsa.QsaShape(T=96, pos0=2050)) == rec(96)
    assert qsa.qsa_flash_workspace_bytes(qsa.QsaShape(T=96, pos0=30000)) == rec(96)
    assert rec(129) == 129 * 4 * 24 * 258 * 4
    assert qsa.qsa_flash_workspace_bytes(qsa.QsaShape(T=129, pos0=30000)) == rec(129)
    assert qsa.qsa_flash_workspace_bytes(qsa.QsaShape(T=257, pos0=30000)) == 0
    assert qsa.qsa_flash_workspace_bytes(qsa.QsaShape(T=1, pos0=30000)) == 33 * 24 * 258 * 4
    assert qsa.qsa_flash_workspace_bytes(qsa.QsaShape(T=0, pos0=0)) == 0


def test_missing_workspace_is_rejected():
    lib = qsa.load_library()
    A = 0x10000
    s = qsa.QsaShape(T=8, pos0=0)
    E = qsa.QSA_ERR_ARG
    need = qsa.qsa_flash_workspace_bytes(s)
    assert _raw(lib, "qsa_flash", s, A, A, A, A, A, 0, A, 0, 0, 0, None) == E
    assert _raw(lib, "qsa_flash", s, A, A, A, A, A, 0, A, 0, A, need - 1, None) == E
    assert _raw(lib, "qsa_flash", s, A, A, A, A, A, 0, A, 0, A + 16, need, None) == E
    # the two halves of the fused path need the same workspace
    assert _raw(lib, "qsa_flash_prepare", s, A, A, A, A, 0, 0, None) == E
    assert _raw(lib, "qsa_flash_prepare", s, A, A, A, A, A, need - 1, None) == E
    assert _raw(lib, "qsa_flash_attend", s, A, A, A, A, A, 0, A, 0, 0, None) == E
    assert _raw(lib, "qsa_flash_attend", s, A, A, A, A, A, 0, A, A + 16, need, None) == E


def test_part_elems_layout():
    s = qsa.QsaShape(T=4, pos0=8192)
    assert qsa.qsa_part_elems(s) == 4 * 33 * 24 * 258
    assert qsa.qsa_part_elems(qsa.QsaShape(T=0, pos0=0)) == 0


# position of the int64 workspace_bytes argument (after the shape) per entry point
_SIZE_ARG = {"qsa_flash": 9, "qsa_flash_prepare": 5, "qsa_flash_attend": 8}


def _raw(lib, fn, shape, *args):
    cs = shape.c()
    conv = [a if isinstance(a, int) and _SIZE_ARG.get(fn) == i else
            (ctypes.c_void_p(a) if a else None) for i, a in enumerate(args)]
    return getattr(lib, fn)(ctypes.byref(cs), *conv)


@pytest.mark.parametrize("shape,expect", [
    (dict(T=0, pos0=0), qsa.QSA_ERR_SHAPE),
    (dict(T=4, pos0=-1), qsa.QSA_ERR_SHAPE),
    (dict(T=4, pos0=0, n_groups=0), qsa.QSA_ERR_SHAPE),
    (dict(T=4, pos0=10, n_cells=13), qsa.QSA_ERR_SHAPE),
    (dict(T=4, pos0=0, heads_per_group=8), qsa.QSA_ERR_UNSUPPORTED),
    (dict(T=4, pos0=0, head_dim=128), qsa.QSA_ERR_UNSUPPORTED),
    (dict(T=4, pos0=0, budget=0), qsa.QSA_ERR_UNSUPPORTED),
    (dict(T=4, pos0=0, budget=qsa.MAX_BUDGET + 1), qsa.QSA_ERR_UNSUPPORTED),
])
def test_bad_shapes_are_rejected(shape, expect):
    lib = qsa.load_library()
    s = qsa.QsaShape(**shape)
    fake = 0x10000  # never dereferenced: validation fails first
    assert _raw(lib, "qsa_flash", s, fake, fake, fake, fake, fake, fake, fake, None, None, 0,
                None) == expect
    assert _raw(lib, "qsa_topk", s, fake, fake, None) == expect
    assert _raw(lib, "qsa_merge", s, fake, fake, None) == expect
    assert _raw(lib, "qsa_flash_prepare", s, fake, fake, fake, fake, None, 0, None) == expect
    assert _raw(lib, "qsa_flash_attend", s, fake, fake, fake, fake, fake, fake, fake, None, 0,
                None) == expect


def test_null_and_misaligned_pointers_are_rejected():
    lib = qsa.load_library()
    A = 0x10000
    under = qsa.QsaShape(T=8, pos0=0)
    over = qsa.QsaShape(T=8, pos0=2050)
    E = qsa.QSA_ERR_ARG
    # q, kq, ksc, vq, vsc, ids, out, part, workspace, workspace_bytes
    assert _raw(lib, "qsa_flash", under, 0, A, A, A, A, 0, A, 0, None, 0, None) == E
    assert _raw(lib, "qsa_flash", under, A + 8, A, A, A, A, 0, A, 0, None, 0, None) == E   # q 16 B
    assert _raw(lib, "qsa_flash", under, A, A, A + 4, A, A, 0, A, 0, None, 0, None) == E   # ksc 8 B
    assert _raw(lib, "qsa_flash", under, A, A, A, A, A, 0, 0, 0, None, 0, None) == E       # no out
    assert _raw(lib, "qsa_flash", over, A, A, A, A, A, 0, A, 0, None, 0, None) == E        # ids needed
    assert _raw(lib, "qsa_flash", over, A, A, A, A, A, A + 2, A, 0, None, 0, None) == E    # ids 4 B
    assert _raw(lib, "qsa_flash", under, A, A, A, A, A, 0, 0, A + 8, None, 0, None) == E   # part 16 B
    # attend: q, kq, ksc, vq, vsc, ids, out, workspace, workspace_bytes
    assert _raw(lib, "qsa_flash_attend", over, 0, A, A, A, A, A, A, None, 0, None) == E  # q
    assert _raw(lib, "qsa_flash_attend", over, A, A, A, A, A, 0, A, None, 0, None) == E  # ids
    assert _raw(lib, "qsa_flash_attend", over, A, A, A, A, A, A, 0, None, 0, None) == E  # out
    assert _raw(lib, "qsa_flash_prepare", under, A + 4, A, A, A, A, 1 << 30, None) == E  # kq
    assert _raw(lib, "qsa_topk", over, 0, A, None) == E                           # scores
    assert _raw(lib, "qsa_topk", under, 0, 0, None) == E                          # ids
    assert _raw(lib, "qsa_merge", under, A, A + 2, None) == E
    assert _raw(lib, "qsa_merge", under, 0, A, None) == E


def test_quantize_arguments_are_validated():
    lib = qsa.load_library()
    A = 0x10000
    q = lambda rows, dim, x, c, s: lib.qsa_quantize(rows, dim, ctypes.c_void_p(x) if x else None,
                                                     ctypes.c_void_p(c) if c else None,
                                                     ctypes.c_void_p(s) if s else None, None)
    assert q(0, 256, 0, 0, 0) == qsa.QSA_OK                       # nothing to do
    assert q(4, 128, A, A, A) == qsa.QSA_ERR_UNSUPPORTED
    assert q(-1, 256, A, A, A) == qsa.QSA_ERR_SHAPE
    assert q(4, 256, 0, A, A) == qsa.QSA_ERR_ARG                  # x
    assert q(4, 256, A + 8, A, A) == qsa.QSA_ERR_ARG              # x 16 B
    assert q(4, 256, A, A + 4, A) == qsa.QSA_ERR_ARG              # codes 16 B
    assert q(4, 256, A, A, A + 1) == qsa.QSA_ERR_ARG              # scales 2 B
    assert q(4, 256, A, A, 0) == qsa.QSA_ERR_ARG


def test_score_arguments_are_validated():
    lib = qsa.load_library()
    A = 0x10000
    under = qsa.QsaShape(T=8, pos0=0)
    over = qsa.QsaShape(T=8, pos0=2050)
    assert qsa.MAX_INDEX_DIM == _header_defines()["QSA_MAX_INDEX_DIM"]

    def sc(shape, dim, qi, po, out):
        cs = shape.c()
        v = lambda x: ctypes.c_void_p(x) if x else None
        return lib.qsa_score(ctypes.byref(cs), dim, v(qi), v(po), v(out), None)

    assert sc(under, 4, 0, 0, 0) == qsa.QSA_OK                    # no row reads scores
    for dim in (0, 2, 6, qsa.MAX_INDEX_DIM + 4):
        assert sc(over, dim, A, A, A) == qsa.QSA_ERR_UNSUPPORTED
    assert sc(qsa.QsaShape(T=0, pos0=0), 4, A, A, A) == qsa.QSA_ERR_SHAPE
    assert sc(over, 4, 0, A, A) == qsa.QSA_ERR_ARG                # qidx
    assert sc(over, 4, A, 0, A) == qsa.QSA_ERR_ARG                # pooled
    assert sc(over, 4, A, A, 0) == qsa.QSA_ERR_ARG                # scores
    assert sc(over, 4, A + 8, A, A) == qsa.QSA_ERR_ARG            # 16 B alignment
    assert sc(over, 4, A, A + 4, A) == qsa.QSA_ERR_ARG
    assert sc(over, 4, A, A, A + 4) == qsa.QSA_ERR_ARG


def test_page_case_lists_hold_the_pages_counts():
    # the GPU parity tests take their cases from these lists: the r9 result's
    # 13 byte-checked cases, the r14 16-case grid, the r27 40-case matrix
    g = json.load(open(GOLDEN))
    assert len(g["cases_r9_bitwise"]["value"]) == 13
    grid = g["cases_r14_grid"]["value"]
    assert len(grid["T"]) * len(grid["pos0"]) == 16
    dm = g["cases_r27_decode"]["value"]
    assert len(dm["pos"]) * len(dm["tokens"]) == 40


def test_noalloc_checks_arguments_and_scratch_size_on_the_host():
    # qsa_flash_noalloc: q, kq, ksc, vq, vsc, ids, out, part.  Every check
    # below fails before the device is touched (this machine may have none)
    lib = qsa.load_library()
    A = 0x10000
    E = qsa.QSA_ERR_ARG
    under = qsa.QsaShape(T=8, pos0=0)
    over = qsa.QsaShape(T=8, pos0=2050)
    assert _raw(lib, "qsa_flash_noalloc", under, 0, A, A, A, A, 0, A, 0, None) == E   # q
    assert _raw(lib, "qsa_flash_noalloc", under, A, A, A, A, A, 0, 0, 0, None) == E   # out
    assert _raw(lib, "qsa_flash_noalloc", over, A, A, A, A, A, 0, A, 0, None) == E    # ids
    assert _raw(lib, "qsa_flash_noalloc", under, A, A, A + 4, A, A, 0, A, 0, None) == E
    assert _raw(lib, "qsa_flash_noalloc", qsa.QsaShape(T=0, pos0=0), A, A, A, A, A, 0, A, 0,
                None) == qsa.QSA_ERR_SHAPE
    # 4 groups x 1024 chunks of identity prefix need 256 MiB of images
    big = qsa.QsaShape(T=1, pos0=65535, n_groups=4, budget=65536)
    assert qsa.qsa_flash_workspace_bytes(big) > qsa.NOALLOC_SCRATCH_BYTES
    assert _raw(lib, "qsa_flash_noalloc", big, A, A, A, A, A, 0, A, 0, None) == \
        qsa.QSA_ERR_TOO_LARGE
    # the chunk images of 2 groups up to an 8192-cell prefix fill the
    # scratch exactly (qsa_flash_noalloc checks the images only); the full
    # workspace adds room to split that token's one 128-chunk block per
    # group into 3 pieces, which qsa_flash_noalloc then runs whole
    fit = qsa.QsaShape(T=1, pos0=8191, n_groups=2, budget=8192)
    slot = (64 * 256 + 2 * 64) * 4
    assert 2 * 128 * 65536 == qsa.NOALLOC_SCRATCH_BYTES
    assert qsa.qsa_flash_workspace_bytes(fit) == qsa.NOALLOC_SCRATCH_BYTES + 256 + 3 * 2 * slot
    assert qsa.qsa_status_string(qsa.QSA_ERR_TOO_LARGE) != "unknown status"
    assert qsa.qsa_status_string(qsa.QSA_ERR_DEVICE) != "unknown status"


C_PROGRAM = r"""
#include <stdio.h>
#include "qsa.h"
int main(void) {
  qsa_shape s = {96, 2050, 2, QSA_HEADS_PER_GROUP, QSA_HEAD_DIM, QSA_DEFAULT_BUDGET, 2146};
  qsa_shape bad = s;
  bad.T = 0;
  const qsa_f16 *q = 0;
  qsa_f16 *out = 0;
  printf("%lld %lld\n", (long long)qsa_flash_workspace_bytes(&s), (long long)qsa_part_elems(&s));
  printf("%d %d\n", qsa_flash(&s, q, 0, 0, 0, 0, 0, out, 0, 0, 0, 0),
         qsa_flash(&bad, q, 0, 0, 0, 0, 0, out, 0, 0, 0, 0));
  printf("%d %d\n", qsa_quantize(3, 128, 0, 0, 0, 0), qsa_merge(&s, 0, out, 0));
  printf("%s\n", qsa_status_string(QSA_ERR_SHAPE));
  return 0;
}
"""


def test_header_is_plain_c_and_links(tmp_path):
    # a C11 program (gcc, pedantic, warnings as errors) and the same source
    # as C++17 include the header; the C one links libqsa.so and calls it
    # (argument checks only: nothing reaches the GPU)
    lib = qsa.load_library()
    src = tmp_path / "abi.c"
    src.write_text(C_PROGRAM)
    exe = tmp_path / "abi"
    inc = os.path.join(ROOT, "include")
    libdir = os.path.dirname(qsa.LIB_PATH)
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", inc,
                    str(src), "-L", libdir, "-lqsa", "-Wl,-rpath," + libdir, "-o", str(exe)],
                   check=True)
    subprocess.run(["g++", "-std=c++17", "-Wall", "-Wextra", "-pedantic", "-Werror", "-x", "c++",
                    "-I", inc, "-c", str(src), "-o", str(tmp_path / "abi_cpp.o")], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, check=True, timeout=60)
    lines = r.stdout.splitlines()
    s = qsa.QsaShape(T=96, pos0=2050, n_groups=2, n_cells=2146)
    assert lines[0] == "%d %d" % (qsa.qsa_flash_workspace_bytes(s), qsa.qsa_part_elems(s))
    assert lines[1] == "%d %d" % (qsa.QSA_ERR_ARG, qsa.QSA_ERR_SHAPE)
    assert lines[2] == "%d %d" % (qsa.QSA_ERR_UNSUPPORTED, qsa.QSA_ERR_ARG)
    assert lines[3] == lib.qsa_status_string(qsa.QSA_ERR_SHAPE).decode()
