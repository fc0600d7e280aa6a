"""fp64 CPU oracle of one FASA decode step -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
module.  The product path (the HIP library and its Python binding) never
imports, calls or falls back to it, and this module imports nothing from the
product package: the two share no code.

It follows the FASA decode step as the pages define it, in the pages' order and
notation, in plain NumPy float64, one (sequence b, kv head g) unit at a time:

1. TIP -- importance score of every cached token from the dominant FCs only
   (paper-graph-ui review of FASA, section 3.4 "Online Stage 1: Token Importance
   Predictor (TIP)", score equation S_t = sum over i in I_dom of alpha^(i)).
   alpha^(i) for token j is the FC-i dot product of the query with the cached
   key; cached keys are stored after RoPE, so on post-RoPE vectors the FC-i
   contribution is q_{2i} k_{2i} + q_{2i+1} k_{2i+1} (section 3.4 "RoPE from a
   Frequency-Chunk Perspective": the score is an exact sum over FCs).
   Grouped-query attention: the G query heads that share kv head g each add
   their own FC contributions; one score vector per kv head.
2. Forced tokens (optional): the first n_sink and last n_recent cached tokens
   are always kept; the top-B is taken over the remaining tokens.
3. Top-B -- T_t = TopK-I(S_t, N_fac): the indices of the B largest scores
   (section 3.4, token-selection equation; TopK-I is defined with the CA metric
   as "indices of the K largest values").  Largest is signed; equal scores go to
   the lower token index.  B >= candidates keeps every candidate.
4. FAC -- softmax(q K_T^T / sqrt(d)) V_T over the gathered rows, which keep
   their original positions (section 3.4 "Online Stage 2: Focused Attention
   Computation (FAC)", gather and attention equations), for every query head
   of the group.

Pinned against: closed forms of RoPE scores, the exact FC decomposition of the
full dot product, full sorts on small inputs, a library scaled-dot-product
attention (per unit, and for a whole paged multi-head step), exact integer
arithmetic on small inputs, and special cases (see tests/oracle_pins.py).
"""
from __future__ import annotations

import numpy as np

BLOCK = 256


# ---------------------------------------------------------------------------
# inputs: the paged cache as plain rows
# ---------------------------------------------------------------------------
def cache_rows(pool: np.ndarray, block_table_row: np.ndarray, g: int, t: int) -> np.ndarray:
    """Rows 0..t-1 of kv head g, read through a block table.

    pool: [n_blocks][H_kv][256][d]; logical token j lives in physical block
    block_table_row[j // 256], slot j % 256.
    """
    d = pool.shape[-1]
    out = np.empty((t, d), dtype=np.float64)
    for j0 in range(0, t, BLOCK):
        n = min(BLOCK, t - j0)
        out[j0:j0 + n] = pool[int(block_table_row[j0 // BLOCK]), g, :n, :]
    return out


def slab_rows(K: np.ndarray, fc: np.ndarray) -> np.ndarray:
    """The dominant-key cache C_key^dom of one unit: [F][t][2], FC-major.

    Section 3.4 "Hardware-Aware Variants": the dominant key cache holds only the
    dimensions of the dominant FCs of every cached key.  Entry [f][j] is the
    pair (K[j, 2 fc[f]], K[j, 2 fc[f] + 1]); an unused slot (fc[f] < 0, a head
    with fewer dominant FCs than the row has slots) holds zeros.
    """
    F = len(fc)
    out = np.zeros((F, K.shape[0], 2), dtype=K.dtype)
    for f in range(F):
        if int(fc[f]) < 0:
            continue
        out[f, :, 0] = K[:, 2 * fc[f]]
        out[f, :, 1] = K[:, 2 * fc[f] + 1]
    return out


# ---------------------------------------------------------------------------
# 1. TIP
# ---------------------------------------------------------------------------
def tip_scores(q_group: np.ndarray, K: np.ndarray, fc: np.ndarray) -> np.ndarray:
    """S[j] = sum_h sum_{i in I_dom} (q_h[2i] K[j,2i] + q_h[2i+1] K[j,2i+1]).

    q_group: [G][d] post-RoPE queries of the heads sharing this kv head.
    K: [t][d] post-RoPE cached keys.  fc: the dominant FC indices I_dom; entries
    < 0 are unused slots (a head with fewer dominant FCs, per-head N_tip) and
    contribute nothing.
    """
    q_group = np.asarray(q_group, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    S = np.zeros(K.shape[0], dtype=np.float64)
    for h in range(q_group.shape[0]):
        for i in fc:
            i = int(i)
            if i < 0:
                continue
            S += q_group[h, 2 * i] * K[:, 2 * i] + q_group[h, 2 * i + 1] * K[:, 2 * i + 1]
    return S


# ---------------------------------------------------------------------------
# 2-3. forced tokens and TopK-I
# ---------------------------------------------------------------------------
def forced_tokens(t: int, n_sink: int, n_recent: int) -> np.ndarray:
    """{0..n_sink-1} U {t-n_recent..t-1}, clipped to [0, t), ascending."""
    keep = set(range(0, min(n_sink, t))) | set(range(max(0, t - n_recent), t))
    return np.array(sorted(keep), dtype=np.int64)


def top_b(S: np.ndarray, budget: int, exclude: np.ndarray = None):
    """TopK-I(S, B) over the tokens not in ``exclude``.

    Candidates are ordered by (-S[j], j): a larger score first, a lower index
    first among equal scores; the first min(B, |candidates|) are chosen.
    -0.0 and +0.0 compare equal.  Returns (chosen indices ascending, s_B) where
    s_B is the score of the last chosen candidate (None if nothing is chosen).
    """
    t = len(S)
    cand = np.ones(t, dtype=bool)
    if exclude is not None and len(exclude):
        cand[np.asarray(exclude, dtype=np.int64)] = False
    idx = np.nonzero(cand)[0]
    order = np.lexsort((idx, -S[idx]))           # primary -S, secondary j
    n = min(int(budget), len(idx))
    ranked = idx[order[:n]]                      # in rank order
    s_b = float(S[ranked[-1]]) if n else None
    return np.sort(ranked), s_b


def select(S: np.ndarray, budget: int, n_sink: int = 0, n_recent: int = 0):
    """sel = forced U TopK-I(S over the rest, B), ascending; also returns s_B."""
    forced = forced_tokens(len(S), n_sink, n_recent)
    chosen, s_b = top_b(S, budget, forced)
    sel = np.union1d(forced, chosen).astype(np.int64)
    return sel, s_b


# ---------------------------------------------------------------------------
# 4. FAC
# ---------------------------------------------------------------------------
def fac(q_group: np.ndarray, K_sel: np.ndarray, V_sel: np.ndarray, scale: float):
    """O_h = softmax(q_h K_T^T * scale) V_T for every head h of the group.

    Returns (out [G][d], p [G][|T|]).  An empty selection gives zeros.
    """
    q_group = np.asarray(q_group, dtype=np.float64)
    K_sel = np.asarray(K_sel, dtype=np.float64)
    V_sel = np.asarray(V_sel, dtype=np.float64)
    G, d = q_group.shape
    n = K_sel.shape[0]
    if n == 0:
        return np.zeros((G, d)), np.zeros((G, 0))
    z = (q_group @ K_sel.T) * scale                 # [G][n]
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    p = e / e.sum(axis=1, keepdims=True)
    return p @ V_sel, p


# ---------------------------------------------------------------------------
# the whole step
# ---------------------------------------------------------------------------
def decode_unit(q_group, K, V, fc, budget, n_sink=0, n_recent=0, scale=None):
    """TIP -> forced U top-B -> FAC for one (sequence, kv head) unit."""
    d = K.shape[1]
    scale = 1.0 / np.sqrt(d) if not scale else scale
    S = tip_scores(q_group, K, fc)
    sel, s_b = select(S, budget, n_sink, n_recent)
    out, p = fac(q_group, K[sel], V[sel], scale)
    return {"S": S, "sel": sel, "s_B": s_b, "out": out, "p": p}


def decode(q, k_pool, v_pool, block_table, seq_lens, fc_idx, budget,
           n_sink=0, n_recent=0, scale=None, units=None):
    """Every (b, g) unit of one decode step (or only ``units``).

    q: [batch][H_q][d]; pools: [n_blocks][H_kv][256][d]; query head h belongs to
    kv head h // (H_q / H_kv).  Returns {(b, g): decode_unit result}.
    """
    H = k_pool.shape[1]
    Hq = q.shape[1]
    G = Hq // H
    res = {}
    if units is None:
        units = [(b, g) for b in range(q.shape[0]) for g in range(H)]
    for b, g in units:
        t = int(seq_lens[b])
        K = cache_rows(k_pool, block_table[b], g, t)
        V = cache_rows(v_pool, block_table[b], g, t)
        res[(b, g)] = decode_unit(q[b, g * G:(g + 1) * G], K, V, fc_idx[g], budget,
                                  n_sink, n_recent, scale)
    return res


# ---------------------------------------------------------------------------
# offline calibration: Contextual Agreement and the dominant FCs
# ---------------------------------------------------------------------------
def ca_score_vectors(q_group: np.ndarray, K: np.ndarray) -> np.ndarray:
    """The full-head score vector alpha and the 64 single-FC vectors alpha^(i)
    of one unit, [1 + d/2][t] in float64 (review section 3.4, the CA metric:
    raw pre-softmax dot products of the query with every past key, over all of
    q.k for alpha and over FC i's pair of columns for alpha^(i)).

    Grouped-query attention: one vector per kv head, from the group's queries
    summed per column -- by linearity, the sum of the heads' own scores, which
    is the score TIP ranks by.
    """
    q_group = np.asarray(q_group, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    qs = q_group.sum(axis=0)
    d = K.shape[1]
    out = np.empty((1 + d // 2, K.shape[0]), dtype=np.float64)
    out[0] = K @ qs
    for i in range(d // 2):
        out[1 + i] = qs[2 * i] * K[:, 2 * i] + qs[2 * i + 1] * K[:, 2 * i + 1]
    return out


def contextual_agreement(q_group: np.ndarray, K: np.ndarray, k_top: int) -> np.ndarray:
    """CA_K for every FC of one unit, [d/2]: |TopK-I(alpha) n TopK-I(alpha^(i))| / K
    (review section 3.4, the CA equation).  TopK-I is top_b (largest first,
    lower index on ties); with fewer than K tokens it keeps them all."""
    vec = ca_score_vectors(q_group, K)
    full, _ = top_b(vec[0], k_top)
    full = set(full.tolist())
    ca = np.empty(vec.shape[0] - 1)
    for i in range(vec.shape[0] - 1):
        fc_set, _ = top_b(vec[1 + i], k_top)
        ca[i] = len(full & set(fc_set.tolist())) / float(k_top)
    return ca


def dominant_fcs(mean_ca: np.ndarray, n_tip: int) -> np.ndarray:
    """I_dom of one head: the n_tip FCs with the highest mean CA (review section
    3.4, offline calibration: sort by mean CA, take the top N_tip; equal means
    go to the lower FC index), returned in ascending FC order."""
    chosen, _ = top_b(np.asarray(mean_ca, dtype=np.float64), n_tip)
    return np.sort(chosen)


# ---------------------------------------------------------------------------
# FASA-M: the host-resident part of the keys
# ---------------------------------------------------------------------------
def nondominant_rows(K: np.ndarray, fc: np.ndarray) -> np.ndarray:
    """C_key^nondom of one unit: the key columns outside the dominant FC pairs,
    in ascending column order, [t][d - 2F].

    FASA-M keeps only the dominant dimensions of past keys on the GPU and
    offloads the remaining key dimensions, with all values, to host memory
    (review section 3.4, "Hardware-Aware Variants", FASA-M's three-way split of
    the cache).  Together with slab_rows they hold every key column once.
    """
    K = np.asarray(K)
    d = K.shape[1]
    dominant = set()
    for i in np.asarray(fc).tolist():
        dominant.add(2 * int(i))
        dominant.add(2 * int(i) + 1)
    keep = [c for c in range(d) if c not in dominant]
    return K[:, keep]


# ---------------------------------------------------------------------------
# dense decode: the full-KV attention that FASA replaces
# ---------------------------------------------------------------------------
def dense_decode(q, k_pool, v_pool, block_table, seq_lens, scale=None, units=None):
    """Full attention over every cached token, for every query head.

    The full-KV (FKV) reference of the review's experimental section, and the
    standard attention whose loads Equation 8 (section 3.4, "Hardware-Aware
    Variants") counts as 2td elements: out_h = softmax(q_h K^T * scale) V over
    tokens 0..t_b-1 of kv head g(h).  No TIP and no selection.  Returns
    {(b, g): out [G][d]}.
    """
    H = k_pool.shape[1]
    Hq = q.shape[1]
    G = Hq // H
    d = k_pool.shape[-1]
    scale = 1.0 / np.sqrt(d) if not scale else scale
    res = {}
    if units is None:
        units = [(b, g) for b in range(q.shape[0]) for g in range(H)]
    for b, g in units:
        t = int(seq_lens[b])
        K = cache_rows(k_pool, block_table[b], g, t)
        V = cache_rows(v_pool, block_table[b], g, t)
        res[(b, g)] = fac(q[b, g * G:(g + 1) * G], K, V, scale)[0]
    return res
