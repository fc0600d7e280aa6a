"""Byte and flop model of one FASA decode step (used by the benchmark's roofline).

Memory-movement model of FASA-C (paper-graph-ui review of FASA, section 3.4
"Hardware-Aware Variants", FASA-C paragraph, and "Efficiency Analysis", memory
movement): standard decode attention reads 2 t d cache elements per head; FASA
reads t * d_dom elements in TIP (d_dom = 2 N_tip) plus 2 N_fac d in FAC, so the
fraction loaded is N_tip/d + N_fac/t, and Equation 8 bounds the speedup by
1 / (N_tip/d + N_fac/t).
"""
from __future__ import annotations

import numpy as np


def fraction_loaded(n_tip: int, d: int, n_fac: int, t: int) -> float:
    """(t * 2 N_tip + 2 N_fac d) / (2 t d) = N_tip/d + N_fac/t."""
    return (t * 2 * n_tip + 2 * n_fac * d) / (2.0 * t * d)


def eq8_speedup(n_tip: int, d: int, n_fac: int, t: int) -> float:
    """Equation 8: 2 t d / (2 t N_tip + 2 N_fac d)."""
    return (2.0 * t * d) / (2 * t * n_tip + 2 * n_fac * d)


def selected_counts(seq_lens, budget: int, n_sink: int = 0, n_recent: int = 0) -> np.ndarray:
    """|sel| per sequence: forced tokens plus min(B, remaining candidates)."""
    out = []
    for t in np.asarray(seq_lens, dtype=np.int64):
        t = int(t)
        forced = len(set(range(min(n_sink, t))) | set(range(max(0, t - n_recent), t)))
        out.append(forced + min(budget, t - forced))
    return np.array(out, dtype=np.int64)


def step_bytes(seq_lens, n_q_heads: int, n_kv_heads: int, head_dim: int, n_fc: int,
               elem_bytes: int, budget: int, n_sink: int = 0, n_recent: int = 0) -> dict:
    """Algorithmic HBM bytes of one decode step over every (sequence, kv head) unit.

    slab   : the dominant-FC key columns TIP must read, sum_b t_b H_kv 2F e
    rows   : the gathered K and V rows FAC must read, sum_b H_kv |sel_b| 2 d e
    q, out : the query (cache dtype) and the fp32 output
    sel    : the selected index lists (int32)
    scores : the fp32 score vector written by TIP and read back by the select
             (an implementation overhead, not part of the algorithmic total)
    dense  : what full decode attention reads, sum_b 2 t_b H_kv d e
    """
    lens = np.asarray(seq_lens, dtype=np.int64)
    sel = selected_counts(lens, budget, n_sink, n_recent)
    b = len(lens)
    r = {
        "slab": int(lens.sum()) * n_kv_heads * 2 * n_fc * elem_bytes,
        "rows": int(sel.sum()) * n_kv_heads * 2 * head_dim * elem_bytes,
        "q": b * n_q_heads * head_dim * elem_bytes,
        "out": b * n_q_heads * head_dim * 4,
        "sel": int(sel.sum()) * n_kv_heads * 4,
        "scores": 2 * int(lens.sum()) * n_kv_heads * 4,
        "dense": int(lens.sum()) * n_kv_heads * 2 * head_dim * elem_bytes,
    }
    r["algorithmic"] = r["slab"] + r["rows"] + r["q"] + r["out"] + r["sel"]
    return r


def step_flops(seq_lens, n_q_heads: int, n_kv_heads: int, head_dim: int, n_fc: int,
               budget: int, n_sink: int = 0, n_recent: int = 0) -> dict:
    """TIP: 2 * 2F flops per token per kv head (query heads folded first);
    FAC: 4 d flops per selected row per query head (q.k and p.v)."""
    lens = np.asarray(seq_lens, dtype=np.int64)
    sel = selected_counts(lens, budget, n_sink, n_recent)
    return {
        "tip": int(lens.sum()) * n_kv_heads * 4 * n_fc,
        "fac": int(sel.sum()) * n_q_heads * 4 * head_dim,
    }
