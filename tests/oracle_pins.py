"""Pins of the fp64 oracle against what the FASA pages and mathematics fix.

Each ``pin_*`` function takes an oracle module and raises AssertionError if it
disagrees with an independent fact: a closed form, an exact identity the pages
state, a library routine, or a brute-force enumeration.  tests/test_oracle_pins.py
runs every pin on the real oracle; tests/test_oracle_mutants.py plants plausible
mistakes in a copy of the oracle and checks that some pin fails for each.
"""
from __future__ import annotations

import heapq
import itertools
import json
import os

import numpy as np
import torch

from query_aware_sparse_fasa_amd import costmodel, synth

D = 128
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "pages_numbers.json")


def _rope(x: np.ndarray, pos, theta: float) -> np.ndarray:
    return synth.apply_rope(torch.from_numpy(np.asarray(x, dtype=np.float64)),
                            torch.as_tensor(pos, dtype=torch.int64), theta).numpy()


# --------------------------------------------------------------------------- TIP
def pin_tip_closed_form(O):
    """A single FC i with pre-RoPE q = (1,0) at position t and k = (1,0) at
    position j scores cos((t-j) theta_i); q = (0,1) scores sin((t-j) theta_i)
    (rotation of FC i by m theta_i, section 3.4 'RoPE from a Frequency-Chunk
    Perspective').  Every other FC contributes nothing."""
    for theta, t in ((1e4, 4096), (5e5, 32768), (1e6, 131072)):
        j = np.array([0, 1, 7, t // 3, t - 2, t - 1])
        for i in (0, 5, 31, 63):
            ang = (t - j) * theta ** (-2.0 * i / D)
            for comp, expect in ((0, np.cos(ang)), (1, np.sin(ang))):
                q = np.zeros((1, 1, D)); q[0, 0, 2 * i + comp] = 1.0
                k = np.zeros((1, len(j), D)); k[0, :, 2 * i] = 1.0
                qr = _rope(q, [t], theta)[0]              # [1][d]
                kr = np.concatenate([_rope(k[:, n:n + 1], [jj], theta)[0] for n, jj in enumerate(j)])
                S = O.tip_scores(qr, kr, np.array([i]))
                np.testing.assert_allclose(S, expect, atol=1e-9, rtol=0)
                other = [(i + 1) % 64, (i + 17) % 64]
                S0 = O.tip_scores(qr, kr, np.array(other))
                np.testing.assert_allclose(S0, 0.0, atol=1e-12)


def pin_tip_relative_form(O):
    """On post-RoPE vectors the TIP score over a set I equals the pages' relative
    form sum_{i in I} q^[i] R_{t-j, theta_i} k^[i]^T on the pre-RoPE vectors
    (section 3.4, FC decomposition of A_{t1,t2}), for every query head summed."""
    rng = np.random.default_rng(11)
    theta, t, G = 5e5, 3000, 3
    qp = rng.standard_normal((G, 1, D))
    kp = rng.standard_normal((1, 40, D))
    jj = np.sort(rng.choice(t, size=40, replace=False))
    qr = _rope(qp, [t], theta)[:, 0, :]
    kr = np.concatenate([_rope(kp[:, n:n + 1], [int(x)], theta)[0] for n, x in enumerate(jj)])
    I = np.array([2, 9, 10, 33, 50, 63])
    S = O.tip_scores(qr, kr, I)
    ref = np.zeros(len(jj))
    for h in range(G):
        for n, j in enumerate(jj):
            for i in I:
                a = (t - j) * theta ** (-2.0 * i / D)
                R = np.array([[np.cos(a), -np.sin(a)], [np.sin(a), np.cos(a)]])
                ref[n] += qp[h, 0, 2 * i:2 * i + 2] @ R @ kp[0, n, 2 * i:2 * i + 2]
    np.testing.assert_allclose(S, ref, rtol=1e-10, atol=1e-10)


def pin_tip_all_fc_is_full_dot(O):
    """With every FC dominant, the score is the full dot product summed over the
    group's query heads (the FC decomposition is exact)."""
    rng = np.random.default_rng(12)
    for G in (1, 4, 7):
        q = rng.standard_normal((G, D)) * 3
        K = rng.standard_normal((257, D))
        S = O.tip_scores(q, K, np.arange(64))
        ref = np.matmul(K, q.sum(axis=0))
        np.testing.assert_allclose(S, ref, rtol=1e-12, atol=1e-10)
        # a subset: the matmul restricted to the FC's columns
        I = np.array([0, 3, 63, 40])
        cols = np.sort(np.concatenate([2 * I, 2 * I + 1]))
        ref = np.matmul(K[:, cols], q[:, cols].sum(axis=0))
        np.testing.assert_allclose(O.tip_scores(q, K, I), ref, rtol=1e-12, atol=1e-10)


def pin_tip_reads_only_dominant(O):
    """Changing non-dominant key dimensions leaves S unchanged; changing one
    dominant dimension changes it."""
    rng = np.random.default_rng(13)
    q = rng.standard_normal((2, D)); K = rng.standard_normal((50, D))
    I = np.array([4, 20])
    S = O.tip_scores(q, K, I)
    K2 = K.copy()
    mask = np.ones(D, bool); mask[[8, 9, 40, 41]] = False
    K2[:, mask] = rng.standard_normal((50, int(mask.sum())))
    np.testing.assert_array_equal(O.tip_scores(q, K2, I), S)
    K3 = K.copy(); K3[:, 41] += 1.0
    assert np.all(O.tip_scores(q, K3, I) != S)


# --------------------------------------------------------------------------- top-B
def _sorted_topb(S, B, excl=()):
    cand = [j for j in range(len(S)) if j not in set(excl)]
    return sorted(sorted(cand, key=lambda j: (-S[j], j))[:B])


def pin_topb_full_sort(O):
    """TopK-I equals a full sort by (-S, j) on small inputs, with heavy ties and
    negative values; heapq.nlargest gives the same set."""
    rng = np.random.default_rng(14)
    for trial in range(60):
        t = int(rng.integers(1, 65))
        S = rng.integers(-4, 5, size=t).astype(np.float64) * (0.5 if trial % 2 else 1.3)
        if trial % 3 == 0:
            S = rng.standard_normal(t)
        for B in (1, 2, t // 2, t - 1, t, t + 5):
            if B < 1:
                continue
            sel, s_b = O.top_b(S, B)
            assert list(sel) == _sorted_topb(S, B)
            nl = heapq.nlargest(min(B, t), ((S[j], -j) for j in range(t)))
            assert sorted(-x[1] for x in nl) == list(sel)
            assert s_b == nl[-1][0]


def pin_topb_exhaustive(O):
    """For t <= 9 and every score pattern over {0, 1, 2}: no excluded token has a
    larger score than an included one, and among equal scores the included ones
    have the lower indices (the tie rule)."""
    for t in range(1, 8):
        for S in itertools.product((0.0, 1.0, 2.0), repeat=t):
            S = np.array(S)
            for B in range(1, t + 1):
                sel, _ = O.top_b(S, B)
                assert len(sel) == B and len(set(sel.tolist())) == B
                inc = set(sel.tolist())
                for a in inc:
                    for b in range(t):
                        if b in inc:
                            continue
                        assert S[a] > S[b] or (S[a] == S[b] and a < b)


def pin_topb_signed_and_zero(O):
    """Largest is signed (not |S|), and -0.0 ties with +0.0."""
    S = np.array([-5.0, 1.0, -0.5, 0.25])
    assert list(O.top_b(S, 1)[0]) == [1]
    assert list(O.top_b(S, 3)[0]) == [1, 2, 3]
    Z = np.array([-0.0, 0.0, -0.0, 0.0])
    assert list(O.top_b(Z, 2)[0]) == [0, 1]


def pin_forced_union(O):
    """Forced tokens (first n_sink, last n_recent) are always selected and the
    budget B is spent on the best of the remaining tokens."""
    rng = np.random.default_rng(15)
    for t, ns, nr, B in ((100, 4, 10, 20), (12, 4, 64, 5), (70, 4, 64, 512), (9, 0, 3, 2),
                         (300, 4, 64, 512), (5, 2, 0, 1)):
        S = rng.standard_normal(t)
        forced = sorted(set(range(min(ns, t))) | set(range(max(0, t - nr), t)))
        assert list(O.forced_tokens(t, ns, nr)) == forced
        sel, _ = O.select(S, B, ns, nr)
        expect = sorted(set(forced) | set(_sorted_topb(S, B, forced)))
        assert list(sel) == expect
        assert len(sel) == len(forced) + min(B, t - len(forced))


# --------------------------------------------------------------------------- FAC
def pin_fac_is_library_attention(O):
    """With all FCs dominant and B >= t the whole step is textbook attention:
    torch's scaled_dot_product_attention in fp64 over every cached token."""
    rng = np.random.default_rng(16)
    for G, t in ((1, 37), (4, 300), (7, 129)):
        q = rng.standard_normal((G, D)) * 2
        K = rng.standard_normal((t, D)) * 2
        V = rng.standard_normal((t, D))
        r = O.decode_unit(q, K, V, np.arange(64), budget=t + 3)
        assert list(r["sel"]) == list(range(t))
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None, :, None, :], torch.from_numpy(K)[None, None].expand(1, G, t, D),
            torch.from_numpy(V)[None, None].expand(1, G, t, D))[0, :, 0, :].numpy()
        np.testing.assert_allclose(r["out"], ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(r["p"].sum(axis=1), 1.0, rtol=0, atol=1e-12)
        assert (r["p"] >= 0).all()


def pin_fac_special_cases(O):
    """B = 1 gives exactly V[sel]; identical key rows give the mean of the
    selected values; the result does not depend on the order of the rows;
    scale 1/sqrt(d) is the default."""
    rng = np.random.default_rng(17)
    q = rng.standard_normal((2, D)); K = rng.standard_normal((64, D)); V = rng.standard_normal((64, D))
    r = O.decode_unit(q, K, V, np.array([1, 2, 3]), budget=1)
    assert len(r["sel"]) == 1
    np.testing.assert_array_equal(r["out"], np.repeat(V[r["sel"]], 2, axis=0))
    Kc = np.repeat(K[:1], 64, axis=0)
    out, p = O.fac(q, Kc[:10], V[:10], 1 / np.sqrt(D))
    np.testing.assert_allclose(out, np.repeat(V[:10].mean(axis=0)[None], 2, axis=0), rtol=1e-12, atol=1e-12)
    perm = rng.permutation(20)
    a, _ = O.fac(q, K[:20], V[:20], 0.1)
    b, _ = O.fac(q, K[:20][perm], V[:20][perm], 0.1)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)
    # scale: two rows whose logits differ by s * sqrt(d) have weights in ratio e^s
    q1 = np.zeros((1, D)); q1[0, 0] = 1.0
    K2 = np.zeros((2, D)); K2[0, 0] = np.sqrt(D); K2[1, 0] = 0.0
    _, p = O.fac(q1, K2, np.eye(2, D), 1 / np.sqrt(D))
    np.testing.assert_allclose(p[0, 0] / p[0, 1], np.e, rtol=1e-12)
    r = O.decode_unit(q1, K2, np.eye(2, D), np.arange(64), budget=2)
    np.testing.assert_allclose(r["p"][0, 0] / r["p"][0, 1], np.e, rtol=1e-12)


def pin_fac_duplicate_keys_tie(O):
    """Duplicate cached keys score exactly equal in TIP, and the tie goes to the
    lower index."""
    rng = np.random.default_rng(18)
    K = rng.standard_normal((30, D)); V = rng.standard_normal((30, D))
    q = rng.standard_normal((1, D))
    S = O.tip_scores(q, K, np.arange(0, 64, 4))
    top = int(np.argmax(S))
    K[[3, 17, 25]] = K[top]
    r = O.decode_unit(q, K, V, np.arange(0, 64, 4), budget=2)
    dup = sorted({3, 17, 25, top})
    assert list(r["sel"]) == dup[:2]


# --------------------------------------------------------------------------- paging
def pin_paged_rows(O):
    """Reading the cache through a permuted block table returns the logical rows
    in order: each row carries its own (b, g, j) in its first three elements."""
    rng = np.random.default_rng(19)
    lens = [700, 256, 1, 513]
    H = 3
    nblk = [(t + 255) // 256 for t in lens]
    perm = rng.permutation(sum(nblk))
    pool = np.full((sum(nblk) + 1, H, 256, 8), np.nan)
    table = np.full((len(lens), max(nblk)), sum(nblk), dtype=np.int32)
    o = 0
    for b, t in enumerate(lens):
        table[b, :nblk[b]] = perm[o:o + nblk[b]]
        o += nblk[b]
        for g in range(H):
            for j in range(t):
                pool[table[b, j // 256], g, j % 256, :3] = (b, g, j)
    for b, t in enumerate(lens):
        for g in range(H):
            rows = O.cache_rows(pool, table[b], g, t)
            np.testing.assert_array_equal(rows[:, 0], b)
            np.testing.assert_array_equal(rows[:, 1], g)
            np.testing.assert_array_equal(rows[:, 2], np.arange(t))


def pin_dense_is_library_attention(O):
    """Dense decode over a paged cache (permuted block table, ragged lengths
    including 0 and 1) equals torch's scaled_dot_product_attention in fp64 on
    the logical rows, head by head of each group; t = 0 gives zeros."""
    rng = np.random.default_rng(21)
    lens = [300, 0, 1, 513]
    H, G = 2, 3
    nblk = [(t + 255) // 256 for t in lens]
    perm = rng.permutation(sum(nblk))
    kp = np.full((sum(nblk) + 1, H, 256, D), np.nan)
    vp = np.full_like(kp, np.nan)
    table = np.full((len(lens), max(max(nblk), 1)), sum(nblk), dtype=np.int32)
    q = rng.standard_normal((len(lens), H * G, D)) * 1.5
    rows = {}
    o = 0
    for b, t in enumerate(lens):
        table[b, :nblk[b]] = perm[o:o + nblk[b]]
        o += nblk[b]
        for g in range(H):
            K = rng.standard_normal((t, D)) * 1.5
            V = rng.standard_normal((t, D))
            rows[(b, g)] = (K, V)
            for j in range(t):
                kp[table[b, j // 256], g, j % 256] = K[j]
                vp[table[b, j // 256], g, j % 256] = V[j]
    res = O.dense_decode(q, kp, vp, table, np.array(lens))
    for (b, g), (K, V) in rows.items():
        t = lens[b]
        qg = q[b, g * G:(g + 1) * G]
        if t == 0:
            np.testing.assert_array_equal(res[(b, g)], 0.0)
            continue
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qg)[None, :, None, :], torch.from_numpy(K)[None, None].expand(1, G, t, D),
            torch.from_numpy(V)[None, None].expand(1, G, t, D))[0, :, 0, :].numpy()
        np.testing.assert_allclose(res[(b, g)], ref, rtol=1e-12, atol=1e-12)


def pin_decode_is_library_attention(O):
    """The whole step over a paged, multi-head cache (permuted block table,
    ragged lengths, three kv heads of two query heads each): with every FC
    dominant and B >= t it is torch's scaled_dot_product_attention in fp64 on
    the logical rows, for each group's own query heads."""
    rng = np.random.default_rng(22)
    lens = [5, 300, 260]
    H, G = 3, 2
    nblk = [(t + 255) // 256 for t in lens]
    perm = rng.permutation(sum(nblk))
    kp = np.full((sum(nblk) + 1, H, 256, D), np.nan)
    vp = np.full_like(kp, np.nan)
    table = np.full((len(lens), max(nblk)), sum(nblk), dtype=np.int32)
    q = rng.standard_normal((len(lens), H * G, D))
    rows = {}
    o = 0
    for b, t in enumerate(lens):
        table[b, :nblk[b]] = perm[o:o + nblk[b]]
        o += nblk[b]
        for g in range(H):
            K = rng.standard_normal((t, D))
            V = rng.standard_normal((t, D))
            rows[(b, g)] = (K, V)
            for j in range(t):
                kp[table[b, j // 256], g, j % 256] = K[j]
                vp[table[b, j // 256], g, j % 256] = V[j]
    fc = np.tile(np.arange(D // 2), (H, 1))
    res = O.decode(q, kp, vp, table, np.array(lens), fc, budget=1000)
    for (b, g), (K, V) in rows.items():
        t = lens[b]
        r = res[(b, g)]
        assert list(r["sel"]) == list(range(t))
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[b, g * G:(g + 1) * G])[None, :, None, :],
            torch.from_numpy(K)[None, None].expand(1, G, t, D),
            torch.from_numpy(V)[None, None].expand(1, G, t, D))[0, :, 0, :].numpy()
        np.testing.assert_allclose(r["out"], ref, rtol=1e-12, atol=1e-12)


def pin_decode_per_head_fc_rows(O):
    """Each kv head ranks by its own row of dominant FCs: head g keeps only FC
    a_g, every head's keys carry a planted set of large values in the columns
    of every a_h, a different set per (g, h), and the query weights only the
    first column of each FC -- so head g must select exactly its set (g, g)."""
    rng = np.random.default_rng(23)
    H, G, t, B = 3, 2, 300, 12
    a = [5, 17, 40]
    kp = np.zeros((2, H, 256, D))
    vp = rng.standard_normal((2, H, 256, D))
    table = np.array([[1, 0]], dtype=np.int32)
    q = np.zeros((1, H * G, D))
    for h in range(H):
        q[0, :, 2 * a[h]] = 1.0
    planted = {}
    perm = rng.permutation(t)
    for g in range(H):
        K = rng.uniform(-0.5, 0.5, (t, D))
        for h in range(H):
            P = perm[(g * H + h) * B:(g * H + h + 1) * B]
            planted[(g, h)] = np.sort(P)
            K[P, 2 * a[h]] = 10.0 + rng.uniform(0, 1, B)
        for j in range(t):
            kp[table[0, j // 256], g, j % 256] = K[j]
    fc = np.array([[a[g], -1] for g in range(H)], dtype=np.int32)
    res = O.decode(q, kp, vp, table, np.array([t]), fc, budget=B)
    for g in range(H):
        assert list(res[(0, g)]["sel"]) == list(planted[(g, g)]), g


def pin_fasa_m_split(O):
    """FASA-M's split of the keys: every column appears exactly once, either in
    the dominant-key cache (slab) or among the non-dominant columns, which keep
    ascending order; rows carry their own (token, column) so the check is by
    coordinates, against explicit set arithmetic."""
    rng = np.random.default_rng(23)
    t = 7
    for F in (1, 5, 16, 64):
        fc = np.sort(rng.choice(D // 2, F, replace=False))
        K = 1000.0 * np.arange(t)[:, None] + np.arange(D)[None, :]
        nd = O.nondominant_rows(K, fc)
        dom = {2 * int(i) for i in fc} | {2 * int(i) + 1 for i in fc}
        expect = sorted(set(range(D)) - dom)
        assert nd.shape == (t, D - 2 * F)
        for j in range(t):
            assert list(nd[j] - 1000.0 * j) == expect
        sl = O.slab_rows(K, fc)                  # [F][t][2]
        cols = sorted(set(sl[:, 0, :].ravel().astype(int).tolist()) | set(nd[0].astype(int).tolist()))
        assert cols == list(range(D))


def _exact_topk(vals, k):
    """Indices of the k largest of a list of exact numbers, lower index on ties."""
    return set(sorted(range(len(vals)), key=lambda j: (-vals[j], j))[:k])


def pin_ca_exact_small(O):
    """CA on small-integer inputs, where float32 arithmetic is exact: the
    oracle's alpha and alpha^(i) equal integer dot products computed in Python,
    and its CA equals explicit set intersections over those (with K larger
    than t in one case, where TopK-I keeps every token and CA divides by K)."""
    rng = np.random.default_rng(25)
    for G, t, k in ((1, 9, 3), (3, 12, 5), (2, 6, 8)):
        q = rng.integers(-3, 4, size=(G, D)).astype(np.float64)
        K = rng.integers(-3, 4, size=(t, D)).astype(np.float64)
        qs = [int(sum(q[h, c] for h in range(G))) for c in range(D)]
        vec = O.ca_score_vectors(q, K)
        full = [sum(qs[c] * int(K[j, c]) for c in range(D)) for j in range(t)]
        assert vec[0].tolist() == full
        top_full = _exact_topk(full, k)
        ca = O.contextual_agreement(q, K, k)
        for i in range(D // 2):
            fc = [qs[2 * i] * int(K[j, 2 * i]) + qs[2 * i + 1] * int(K[j, 2 * i + 1]) for j in range(t)]
            assert vec[1 + i].tolist() == fc
            assert ca[i] == len(top_full & _exact_topk(fc, k)) / k


def pin_ca_fc_sum_is_full(O):
    """The 64 single-FC vectors add up to the full-head vector (the FC
    decomposition of the dot product is exact, section 3.4), on random
    inputs with several query heads."""
    rng = np.random.default_rng(24)
    q = rng.standard_normal((3, D)) * 2
    K = rng.standard_normal((40, D)) * 2
    vec = O.ca_score_vectors(q, K)
    assert vec.shape == (1 + D // 2, 40)
    np.testing.assert_allclose(vec[1:].sum(axis=0), vec[0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(vec[0], K @ q.sum(axis=0), rtol=1e-12, atol=1e-12)


def pin_ca_single_fc_query(O):
    """A query that lives in one FC: that FC agrees with the head completely
    (CA 1); every other FC scores all tokens 0, so its top-K is the K lowest
    indices and its CA is their share of the head's top-K."""
    rng = np.random.default_rng(26)
    t, k, i0 = 300, 16, 11
    q = np.zeros((1, D))
    q[0, 2 * i0], q[0, 2 * i0 + 1] = 1.5, -0.75
    K = rng.standard_normal((t, D))
    ca = O.contextual_agreement(q, K, k)
    assert ca[i0] == 1.0
    full = O.ca_score_vectors(q, K)[0].astype(np.float64).tolist()
    share = len(_exact_topk(full, k) & set(range(k))) / k
    assert all(ca[i] == share for i in range(D // 2) if i != i0)


def pin_dominant_fcs(O):
    """The N_tip FCs of highest mean CA, ties to the lower FC index, ascending."""
    m = np.zeros(D // 2)
    m[[40, 3, 17, 60, 9]] = [0.9, 0.5, 0.5, 0.7, 0.5]
    assert list(O.dominant_fcs(m, 3)) == [3, 40, 60]
    assert list(O.dominant_fcs(m, 4)) == [3, 9, 40, 60]
    assert list(O.dominant_fcs(m, 64)) == list(range(64))


def pin_per_head_fc_padding(O):
    """Per-head N_tip: a row of FC indices padded with -1 scores exactly as its
    valid prefix (closed form: with unit query pairs only on the valid FCs, S is
    their key pairs' sum), and the padded slab slots are zero."""
    rng = np.random.default_rng(27)
    K = rng.standard_normal((50, D))
    q = np.zeros((2, D))
    valid = [5, 9, 33]
    for i in valid:
        q[0, 2 * i] = 1.0
        q[1, 2 * i + 1] = 1.0
    for i in (1, 2, 60, 63):                    # FCs present in q but not in the row
        q[0, 2 * i] = 7.0
        q[1, 2 * i + 1] = -3.0
    S = O.tip_scores(q, K, np.array(valid + [-1, -1]))
    expect = sum(K[:, 2 * i] + K[:, 2 * i + 1] for i in valid)
    np.testing.assert_allclose(S, expect, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(S, O.tip_scores(q, K, np.array(valid)))
    sl = O.slab_rows(K, np.array([7, -1]))
    assert (sl[1] == 0).all() and (sl[0, :, 0] == K[:, 14]).all()


def pin_slab(O):
    """The dominant-key cache holds exactly the FC pairs of every key."""
    K = np.arange(5 * D, dtype=np.float64).reshape(5, D)
    fc = np.array([0, 7, 63])
    s = O.slab_rows(K, fc)
    for f, i in enumerate(fc):
        for j in range(5):
            assert s[f, j, 0] == j * D + 2 * i and s[f, j, 1] == j * D + 2 * i + 1


ALL_PINS = [pin_tip_closed_form, pin_tip_relative_form, pin_tip_all_fc_is_full_dot,
            pin_tip_reads_only_dominant, pin_topb_full_sort, pin_topb_exhaustive,
            pin_topb_signed_and_zero, pin_forced_union, pin_fac_is_library_attention,
            pin_fac_special_cases, pin_fac_duplicate_keys_tie, pin_paged_rows, pin_slab,
            pin_dense_is_library_attention, pin_decode_is_library_attention, pin_decode_per_head_fc_rows, pin_fasa_m_split,
            pin_ca_exact_small, pin_ca_fc_sum_is_full, pin_ca_single_fc_query, pin_dominant_fcs,
            pin_per_head_fc_padding]


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def check_costmodel_against_pages():
    """The byte model reproduces the numbers the pages print."""
    g = golden()
    e = g["fraction_loaded_worked_example"]
    v = costmodel.fraction_loaded(e["n_tip"], e["d"], e["n_fac"], e["t"])
    assert round(v, e["digits"]) == e["value"], v
    a = g["fraction_loaded_asymptote"]
    assert abs(costmodel.fraction_loaded(a["n_tip"], a["d"], 0, 10**9) - a["value"]) < 1e-12
    s = g["eq8_speedup_bound"]
    assert abs(costmodel.eq8_speedup(s["n_tip"], s["d"], 0, 10**9) - s["value"]) < 1e-9
    assert abs(costmodel.eq8_speedup(16, 128, 256, 10000) - 1 / v) < 1e-12
    f = g["tip_flop_reduction"]
    assert f["d"] / (2 * f["n_tip"]) == f["value"]
    fs = g["fac_speedup_example"]
    assert round(fs["t"] / fs["n_fac"]) == fs["value"]
    st = g["fc_index_storage"]
    assert st["layers"] * st["heads"] * st["n_tip"] == st["value"]
