"""Host-side logic of bench.py (CPU only): the algorithmic work it divides
by, the traffic-record lookup, and the one-GPU contract."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_algorithmic_work_at_the_headline():
    # T=1984 at pos0 0: token t sees t + 1 cells in each of 2 groups
    visits, by, flops = bench.algorithmic(1984, 0, 2051)
    assert visits == 2 * 1984 * 1985 // 2 == 3938240
    # 528 B of codes and scales per visit, Q and O rows of 12 x 256 fp16
    assert by == visits * 528 + 1984 * 2 * 2 * 12 * 256 * 2
    assert flops == visits * 12 * 256 * 2 * 2
    assert round(flops / 1e9, 2) == 48.39


def test_algorithmic_work_at_long_context():
    # T=1984 at pos0 30000: every token above budget takes 2051 cells and
    # reads 2051 ids per group
    visits, by, flops = bench.algorithmic(1984, 30000, 2051)
    assert visits == 1984 * 2 * 2051 == 8138368
    assert by == visits * (528 + 4) + 1984 * 2 * 12288
    assert round(by / 1e6, 1) == 4378.4


def test_algorithmic_work_across_the_budget():
    # T=96 at pos0 2050: token 0 sees 2051 cells (identity), the rest 2051
    # selected ones with ids
    visits, by, _ = bench.algorithmic(96, 2050, 2051)
    assert visits == 96 * 2 * 2051
    assert by == visits * 528 + 95 * 2 * 2051 * 4 + 96 * 2 * 12288


def test_traffic_records_parse_and_match_their_workloads():
    for wl, names in bench.TRAFFIC_SOURCES.items():
        path = os.path.join(ROOT, "profiles", "traffic_%s.txt" % wl)
        with open(path) as f:
            rec = json.loads([line for line in f if line.startswith("{")][-1])
        assert rec["workload"] == wl
        assert rec["hbm_bytes_per_launch"] == pytest.approx(
            rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"], rel=1e-9)
        # a record taken on other kernel sources is not reported
        value = bench.measured_traffic(wl)
        if rec["kernel_sources_sha256"] == bench.kernel_source_hash(names):
            assert value == rec["hbm_bytes_per_launch"]
        else:
            assert value is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_fused_kernel_labels_follow_the_routes():
    assert bench.fused_kernels(1984, 0, 2051) == \
        "dequant_chunks_kernel + flash_tile_kernel<8>"
    assert bench.fused_kernels(512, 0, 2051) == \
        "dequant_chunks_kernel + flash_tile_kernel<4>"
    # at most 256 rows: every token as row pieces
    assert bench.fused_kernels(96, 2050, 2051).startswith("row pieces")
    # tokens under budget tiled, up to 512 rows above as pieces, else a row
    # per wavefront
    assert bench.fused_kernels(200, 1900, 2051) == \
        "dequant_chunks_kernel + flash_tile_kernel<4> + " + bench.fused_kernels(96, 2050, 2051)
    assert bench.fused_kernels(200, 30000, 2051).startswith("row pieces")
    assert bench.fused_kernels(1984, 30000, 2051) == "flash_rows_staged_kernel<false, false>"
