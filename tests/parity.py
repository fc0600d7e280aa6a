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
* slab, top-B on given scores: bit-exact.
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
