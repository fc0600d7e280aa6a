"""Host-side checks of the benchmark: its byte model and its one-GPU contract (no GPU needed).

The byte model is what the roofline's `achieved` divides by the kernel time, so
it is checked against the counts written out by hand from the definitions:
TIP reads t * H_kv * 2F elements of the dominant key columns, FAC reads
|sel| * H_kv rows of K and of V, full decode attention reads 2 t H_kv d
elements (paper-graph-ui review of FASA, section 3.4 "Efficiency Analysis").
"""
import os
import subprocess
import sys

import numpy as np

from query_aware_sparse_fasa_amd import costmodel, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_step_bytes_llama3_8b_layer():
    # 32768 cached tokens, 8 kv heads, 16 dominant FCs (32 columns) of 2-byte
    # elements; 256 selected rows of 128 channels, K and V; 32 query heads.
    b = costmodel.step_bytes([32768], 32, 8, 128, 16, 2, 256)
    assert b["slab"] == 32768 * 8 * 32 * 2 == 16_777_216
    assert b["rows"] == 8 * 256 * 2 * 128 * 2 == 1_048_576
    assert b["q"] == 32 * 128 * 2
    assert b["out"] == 32 * 128 * 4
    assert b["sel"] == 8 * 256 * 4
    assert b["dense"] == 2 * 32768 * 8 * 128 * 2 == 134_217_728
    assert b["algorithmic"] == 17_858_560


def test_step_bytes_batch16_and_budget_fraction():
    # 18.9% of 32768 tokens, rounded to the nearest token, is the batch-16 budget.
    cfg = synth.CONFIGS["c3"]
    assert cfg.budget == round(0.189 * 32768) == 6193
    b = costmodel.step_bytes([32768] * 16, 32, 8, 128, 16, 2, cfg.budget)
    assert b["slab"] == 16 * 16_777_216
    assert b["rows"] == 16 * 8 * 6193 * 2 * 128 * 2 == 405_864_448


def test_selected_counts_forced_union():
    # 4 first and 64 last tokens are kept on top of the budget; short sequences
    # keep everything; a budget above the candidates keeps every candidate.
    n = costmodel.selected_counts([65536, 600, 500, 68, 10], 512, n_sink=4, n_recent=64)
    assert n.tolist() == [512 + 68, 512 + 68, 500, 68, 10]
    assert costmodel.selected_counts([100], 1000).tolist() == [100]
    assert costmodel.selected_counts([0], 5).tolist() == [0]


def test_step_flops_fold_the_query_heads():
    f = costmodel.step_flops([32768], 32, 8, 128, 16, 256)
    assert f["tip"] == 32768 * 8 * 2 * 2 * 16        # 2F multiply-adds per token and kv head
    # 256 rows per kv head, each used by the 4 query heads of its group: 4d flops each.
    assert f["fac"] == 8 * 256 * 4 * 4 * 128


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single" in r.stderr
    assert r.stdout.strip() == ""


def test_workload_lengths_are_seeded():
    cfg = synth.CONFIGS["c5"]
    a = synth.draw_lengths(cfg, 0)
    b = synth.draw_lengths(cfg, 0)
    np.testing.assert_array_equal(a, b)
    assert len(a) == 64 and a.min() >= 4096 and a.max() <= 65536
