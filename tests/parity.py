"""Comparison rules between the HIP path and the fp64 oracle.

Tolerances (stated once, used by every GPU test):
* selected indices: bit-exact, except that the sets may differ in tokens whose
  oracle score lies within 1e-5 relative of the oracle's B-th candidate score
  (such tokens are near ties: fp32 rounding may order them either way);
  sizes must agree exactly and forced tokens are always present;
* outputs: max |out_gpu - out_oracle| <= 2e-3 for bf16 caches, 1e-5 for fp32;
* TIP scores: |S_gpu - S| <= (2F + G + 2) * 2^-24 * sum_c (sum_h |q_h,c|) |k_c|,
  the forward error bound of the fp32 evaluation order (the group's query
  heads summed per column, then 2F fused multiply-adds);
* slab, top-B on given scores: bit-exact;
* CA top-K lists: each of the 65 lists of a unit equals the oracle's fp64
  TopK-I except in tokens whose fp64 score lies within 1e-5 relative of the
  K-th score plus the fp32 forward error bound of both scores (the group's
  heads summed per column, then per FC two products and one add, then the 64
  FC terms added for alpha); the hit counts then equal, bit for bit, the
  intersections of the validated lists.
"""
from __future__ import annotations

import numpy as np

from oracle import fasa_oracle as O

TIE_RTOL = 1e-5
OUT_ATOL = {"bf16": 2e-3, "fp32": 1e-5}
U32 = 2.0 ** -24


def tip_bound(q_group: np.ndarray, K: np.ndarray, fc: np.ndarray) -> np.ndarray:
    cols = np.sort(np.concatenate([2 * fc, 2 * fc + 1]))
    qa = np.abs(q_group[:, cols]).sum(axis=0)
    mag = np.abs(K[:, cols]) @ qa
    G = q_group.shape[0]
    return (2 * len(fc) + G + 2) * U32 * mag + 1e-30


def check_selection(gpu_sel: np.ndarray, ref: dict, t: int, n_sink: int, n_recent: int,
                    where: str = "") -> bool:
    """Returns True when the sets are identical; asserts the near-tie rule otherwise."""
    osel = ref["sel"]
    assert len(gpu_sel) == len(osel), f"{where}: |sel| {len(gpu_sel)} != oracle {len(osel)}"
    assert np.all(np.diff(gpu_sel) > 0), f"{where}: selection not strictly ascending"
    assert gpu_sel.min(initial=0) >= 0 and gpu_sel.max(initial=-1) < max(t, 1), f"{where}: index out of range"
    forced = O.forced_tokens(t, n_sink, n_recent)
    assert np.isin(forced, gpu_sel).all(), f"{where}: forced token missing"
    if np.array_equal(gpu_sel, osel):
        return True
    diff = np.setxor1d(gpu_sel, osel)
    s_b = ref["s_B"]
    S = ref["S"]
    band = np.abs(S[diff] - s_b) <= TIE_RTOL * abs(s_b)
    assert band.all(), (f"{where}: selections differ outside the 1e-5 tie band: "
                        f"{diff[~band][:10]} scores {S[diff[~band]][:10]} vs s_B {s_b}")
    return False


def check_output(gpu_out: np.ndarray, q_group, K, V, gpu_sel, ref: dict, same_set: bool,
                 dtype: str, scale: float, where: str = ""):
    """Compare one unit's output rows.  When the selections are identical the
    oracle's own output is the reference; when they differ inside the tie band
    (several selections are correct) the oracle's FAC is evaluated on the GPU's
    validated selection."""
    if same_set:
        expect = ref["out"]
    else:
        expect, _ = O.fac(q_group, K[gpu_sel], V[gpu_sel], scale)
    err = np.abs(gpu_out - expect).max(initial=0.0)
    assert err <= OUT_ATOL[dtype], f"{where}: max |out - oracle| = {err:.3e} > {OUT_ATOL[dtype]}"
    return err


def _ca_bounds(q_group: np.ndarray, K: np.ndarray) -> np.ndarray:
    """Forward error bounds of the fp32 CA scores, [1 + d/2][t]."""
    G, d = q_group.shape
    prod = np.abs(K) * np.abs(q_group).sum(axis=0)[None, :]
    out = np.empty((1 + d // 2, K.shape[0]))
    out[0] = (G + 66) * U32 * prod.sum(axis=1)
    out[1:] = (G + 2) * U32 * (prod[:, 0::2] + prod[:, 1::2]).T
    return out + 1e-30


def check_ca_lists(gpu_lists: np.ndarray, q_group: np.ndarray, K: np.ndarray, k_top: int,
                   where: str = "") -> tuple[np.ndarray, int]:
    """Validate one unit's 65 GPU top-K lists ([65][cap], -1 padded) against
    the fp64 CA vectors.  Returns the hit counts those lists give and the number
    of lists that differ from the oracle's inside the band."""
    vec = O.ca_score_vectors(q_group, K)
    bnd = _ca_bounds(q_group, K)
    t = K.shape[0]
    n = min(k_top, t)
    sets = []
    differ = 0
    for r in range(vec.shape[0]):
        row = gpu_lists[r]
        got = row[:n]
        assert (row[n:] == -1).all(), f"{where} row {r}: padding"
        assert np.all(np.diff(got) > 0), f"{where} row {r}: list not strictly ascending"
        assert n == 0 or (got[0] >= 0 and got[-1] < t), f"{where} row {r}: index out of range"
        want, s_k = O.top_b(vec[r], k_top)
        if not np.array_equal(got, want):
            differ += 1
            v = vec[r]
            order = np.lexsort((np.arange(t), -v))
            jk = order[n - 1]
            diff = np.setxor1d(got, want)
            band = np.abs(v[diff] - s_k) <= TIE_RTOL * abs(s_k) + bnd[r, diff] + bnd[r, jk]
            assert band.all(), (f"{where} row {r}: lists differ outside the band: {diff[~band][:10]} "
                                f"scores {v[diff[~band]][:10]} vs s_K {s_k}")
        sets.append(set(got.tolist()))
    hits = np.array([len(sets[0] & sets[1 + i]) for i in range(vec.shape[0] - 1)], dtype=np.int32)
    return hits, differ
