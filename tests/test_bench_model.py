"""bench.py's work and bytes model (host arithmetic) against the figures the
pages print and against closed forms."""
import json
import os

import pytest

import bench

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "printed_values.json")


def _golden():
    data = json.load(open(GOLDEN))
    return {k: v for k, v in data.items() if not k.startswith("_")}


@pytest.mark.parametrize("name", sorted(_golden()))
def test_score_matrix_bytes_reproduces_printed_values(name):
    g = _golden()[name]
    assert bench.score_matrix_bytes(g["t_query"], g["t_key"], g["bytes_per_score"]) == g["value"]


def test_printed_approximations_are_consistent():
    g = _golden()
    # 8192^2 is "about 67 million" entries and 128 MiB at 2 bytes
    assert abs(8192 * 8192 - 67e6) / 67e6 < 0.01
    assert g["score_matrix_8192x8192_fp16"]["value"] == 128 * 2**20
    # 4096^2 is "16 million" floats; 64 MiB at 4 bytes
    assert g["score_matrix_4096x4096_fp32"]["value"] == 64 * 2**20
    assert g["score_matrix_4096x4096_2B"]["value"] == 32 * 2**20


def test_visible_pairs_closed_forms():
    assert bench.visible_pairs(8192, 8192, True) == 8192 * 8193 // 2
    assert bench.visible_pairs(300, 200, False) == 60000
    # top-left causal with Nq > Nk: rows past Nk see all Nk keys
    assert bench.visible_pairs(5, 3, True) == 1 + 2 + 3 + 3 + 3
    assert bench.visible_pairs(3, 5, True) == 1 + 2 + 3
    brute = sum(min(i + 1, 37) for i in range(50))
    assert bench.visible_pairs(50, 37, True) == brute


def test_bench_workload_totals():
    flops = bench.algorithmic_flops([8192], [8192], 32, 128, True)
    assert flops == 549822922752
    assert bench.algorithmic_bytes(8192, 8192, 32, 8, 128, 2) == 168820736


def test_multi_gpu_request_exits_with_message(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err
