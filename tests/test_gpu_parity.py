"""Parity of the HIP path (through the C ABI) with the fp64 oracle.  Needs a GPU.

Every case prints its name before touching the GPU so that a failing run names it.
"""
import sys

import numpy as np
import pytest
import torch

import parity as PR
from oracle import fasa_oracle as O
from query_aware_sparse_fasa_amd import fasa, synth
from query_aware_sparse_fasa_amd.synth import unit_rows
from query_aware_sparse_fasa_amd.workload import DeviceLayer

pytestmark = pytest.mark.gpu

C = synth.CONFIGS
SMALL = {
    "c1": C["c1"],
    "c2-ragged": C["c2"].replace(batch=3, t=None, t_range=(1000, 5000)),
    "c3-shape": C["c3"].replace(batch=2, t=None, t_range=(7000, 9000)),
    "c4-ragged": C["c4"].replace(batch=2, t=None, t_range=(3000, 9000)),
    "c5-ragged": C["c5"].replace(batch=4, t_range=(300, 3000)),
    "fp32-gqa4": C["c2"].replace(dtype="fp32", batch=2, t=None, t_range=(700, 2600), budget=100),
    "g16-f5": C["c2"].replace(n_q_heads=32, n_kv_heads=2, n_fc=5, batch=2, t=None,
                              t_range=(1500, 2500), budget=64),
    "g2-f1-sink": C["c2"].replace(n_q_heads=4, n_kv_heads=2, n_fc=1, batch=2, t=None,
                                  t_range=(600, 900), budget=33, n_sink=3, n_recent=5),
    "f32-fc32": C["c2"].replace(n_q_heads=6, n_kv_heads=3, n_fc=32, batch=1, t=None,
                                t_range=(2000, 2000), budget=300),
    "fp32-g7-f64": C["c4"].replace(dtype="fp32", batch=1, t=None, t_range=(1200, 1300), n_fc=64,
                                   budget=77),
    # At least 256 (sequence, kv head) units: the selecting FAC launch then
    # covers several query heads per workgroup (4, 8 and, for fp32 caches, 2).
    "wide-g4": C["c2"].replace(batch=40, t=None, t_range=(300, 700), budget=48),
    "wide-g8-sink": C["c2"].replace(batch=64, n_kv_heads=4, t=None, t_range=(260, 520), budget=40,
                                    n_sink=2, n_recent=9),
    "wide-fp32-g2": C["c2"].replace(dtype="fp32", batch=64, n_q_heads=8, n_kv_heads=4, t=None,
                                    t_range=(300, 600), budget=40),
}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


_cache = {}


def layer_for(name, seed=0, device="cuda"):
    key = (name, seed)
    if key not in _cache:
        cfg = SMALL[name]
        inp = synth.make_inputs(cfg, seed=seed, device="cpu")
        _cache[key] = (inp, DeviceLayer(inp, device=device))
    return _cache[key]


def oracle_units(inp, units=None):
    cfg = inp.cfg
    res = {}
    for b in range(cfg.batch):
        for g in range(cfg.n_kv_heads):
            if units is not None and (b, g) not in units:
                continue
            G = cfg.group
            q = inp.q[b, g * G:(g + 1) * G].double().cpu().numpy()
            K = unit_rows(inp, b, g, inp.k_pool).double().cpu().numpy()
            V = unit_rows(inp, b, g, inp.v_pool).double().cpu().numpy()
            r = O.decode_unit(q, K, V, inp.fc_idx[g], cfg.budget, cfg.n_sink, cfg.n_recent)
            res[(b, g)] = (q, K, V, r)
    return res


# ------------------------------------------------------------------------ slab
@pytest.mark.parametrize("name", list(SMALL))
def test_slab_build_bit_exact(name):
    say(f"[slab_build] {name}")
    inp, L = layer_for(name)
    torch.cuda.synchronize()
    slab = L.slab.cpu()
    cfg = inp.cfg
    for b in range(cfg.batch):
        t = int(inp.seq_lens[b])
        for g in range(cfg.n_kv_heads):
            K = synth.unit_rows(inp, b, g, inp.k_pool)             # cast values, no widening
            ref = O.slab_rows(K.float().numpy(), inp.fc_idx[g])   # [F][t][2]
            n = (t + 255) // 256
            got = slab[b, :n, g]                                  # [n][F][256][2], logical blocks
            got = got.permute(1, 0, 2, 3).reshape(cfg.n_fc, n * 256, 2)[:, :t].float().numpy()
            np.testing.assert_array_equal(got, ref, err_msg=f"{name} b={b} g={g}")


def test_slab_append_writes_one_slot():
    name = "c5-ragged"
    say(f"[slab_append] {name}")
    inp, L = layer_for(name)
    cfg = inp.cfg
    L2 = DeviceLayer(inp, with_slab=True, build_slab=False)
    L2.slab.fill_(float("nan"))
    pos = np.array([int(t) - 1 for t in inp.seq_lens], dtype=np.int32)
    pos[0] = min(257, int(inp.seq_lens[0]) - 1)       # a slot inside a block
    pos[1] = -1                                      # skipped
    fasa.fasa_slab_append(L2.shape, L2.k_pool, L2.block_table, torch.from_numpy(pos).cuda(),
                          L2.fc_idx, L2.slab)
    torch.cuda.synchronize()
    a, ref = L2.slab.cpu(), L.slab.cpu()                 # [batch][max_blocks][H][F][256][2]
    nb = a.shape[1]
    written = np.zeros(a.shape[0] * nb * 256, dtype=bool)
    for b in range(cfg.batch):
        if pos[b] < 0:
            continue
        k, s = int(pos[b]) // 256, int(pos[b]) % 256
        assert torch.equal(a[b, k, :, :, s], ref[b, k, :, :, s]), b
        written[(b * nb + k) * 256 + s] = True
    rest = a.permute(0, 1, 4, 2, 3, 5).reshape(a.shape[0] * nb * 256, -1)[~torch.from_numpy(written)]
    assert torch.isnan(rest.float()).all()


def test_decode_steps_with_append():
    """Three consecutive decode steps: each appends the new token's key and
    value to the cache (pool rows written by the caller, slab by
    fasa_slab_append), grows seq_lens by one and decodes a fresh query;
    every step against the oracle on the grown cache."""
    cfg = C["c5"].replace(batch=3, budget=40, n_sink=2, n_recent=8)
    say("[decode steps with append]")
    inp = synth.make_inputs(cfg, seed=37, seq_lens=[1000, 700, 513])
    L = DeviceLayer(inp, max_t=1003)               # room for the three appended tokens (block 3 of 4)
    rng = np.random.default_rng(37)
    for step in range(3):
        pos = inp.seq_lens.copy()                      # the new token's position per sequence
        for b in range(cfg.batch):
            blk, slot = int(inp.block_table[b, pos[b] // 256]), int(pos[b]) % 256
            for g in range(cfg.n_kv_heads):
                k = torch.from_numpy(rng.standard_normal(128).astype(np.float32)).to(inp.k_pool.dtype)
                v = torch.from_numpy(rng.standard_normal(128).astype(np.float32)).to(inp.v_pool.dtype)
                inp.k_pool[blk, g, slot] = k
                inp.v_pool[blk, g, slot] = v
                L.k_pool[blk, g, slot] = k.cuda()
                L.v_pool[blk, g, slot] = v.cuda()
        fasa.fasa_slab_append(L.shape, L.k_pool, L.block_table, torch.from_numpy(pos).cuda(), L.fc_idx, L.slab)
        inp.seq_lens += 1
        L.seq_lens.copy_(torch.from_numpy(inp.seq_lens))
        q = torch.from_numpy(rng.standard_normal((cfg.batch, cfg.n_q_heads, 128)).astype(np.float32))
        inp.q = q.to(inp.q.dtype)
        L.q.copy_(inp.q.cuda())
        L.out.fill_(float("nan"))
        L.decode()
        _check_decode(inp, L, oracle_units(inp), f"append step {step}")


# ------------------------------------------------------------------------ TIP
@pytest.mark.parametrize("name", list(SMALL))
def test_tip_scores(name):
    say(f"[tip] {name}")
    inp, L = layer_for(name)
    cfg = inp.cfg
    L.scores.fill_(float("nan"))
    L.tip(use_slab=True)
    s_slab = L.scores.clone()
    L.scores.fill_(float("nan"))
    L.tip(use_slab=False)
    s_rows = L.scores.clone()
    torch.cuda.synchronize()
    s_slab, s_rows = s_slab.cpu().numpy(), s_rows.cpu().numpy()
    for (b, g), (q, K, V, r) in oracle_units(inp).items():
        t = int(inp.seq_lens[b])
        got = s_slab[b, g, :t].astype(np.float64)
        # reading the slab or gathering from the key rows: same arithmetic, same bits
        np.testing.assert_array_equal(s_slab[b, g, :t], s_rows[b, g, :t])
        bound = PR.tip_bound(q, K, inp.fc_idx[g])
        err = np.abs(got - r["S"])
        assert (err <= bound).all(), f"{name} b={b} g={g}: max err/bound {np.max(err / bound):.3f}"
        # columns past t_b are untouched
        assert np.isnan(s_slab[b, g, t:]).all()


# ------------------------------------------------------------------------ top-B
TOPK_CASES = [
    # (kind, batch, H, max_t, lens, budget, n_sink, n_recent)
    ("normal", 2, 3, 5000, [5000, 4097], 256, 0, 0),
    ("normal", 1, 2, 32768, [32768], 256, 0, 0),
    ("normal", 1, 1, 40000, [39999], 1024, 0, 0),        # past the LDS-staged size
    ("ties", 2, 2, 3000, [3000, 2999], 100, 0, 0),
    ("ties", 1, 1, 45000, [45000], 5000, 4, 64),
    ("const", 2, 1, 2000, [2000, 1500], 37, 0, 0),
    ("const", 1, 1, 33000, [33000], 999, 0, 0),
    ("signed_zero", 1, 2, 4096, [4096], 300, 0, 0),
    ("wide", 2, 2, 8192, [8192, 8000], 512, 4, 64),
    ("sorted_asc", 1, 2, 1024, [1024], 10, 0, 0),
    ("sorted_desc", 1, 2, 1024, [1000], 10, 0, 0),
    ("normal", 3, 2, 700, [700, 68, 0], 512, 4, 64),     # B >= candidates, t < forced, t = 0
    ("normal", 2, 1, 300, [1, 300], 1, 0, 0),
    ("normal", 1, 1, 6193 * 5, [6193 * 5], 6193, 0, 0),
    # A ragged batch whose select grid exceeds 2048 workgroups (32 chunks x 8 heads
    # x 9 sequences): the histogram and filter launches read each sequence's length
    # before its scores and skip chunks past its end; lengths at chunk edges and 0.
    ("normal", 9, 8, 65536, [65536, 100, 2047, 2048, 2049, 30000, 4096, 0, 65000], 512, 4, 64),
]


@pytest.mark.parametrize("case", TOPK_CASES, ids=lambda c: f"{c[0]}-t{c[3]}-B{c[5]}")
def test_topk_exact_on_given_scores(case):
    kind, batch, H, max_t, lens, budget, ns, nr = case
    say(f"[topk] {case}")
    scores = synth.random_scores(batch * H, max_t, kind, seed=max_t + budget).reshape(batch, H, max_t)
    shape = fasa.make_shape(batch, H, H, 16, budget, (max_t + 255) // 256, torch.bfloat16, ns, nr)
    cap = fasa.fasa_selection_capacity(shape, max_t)
    dev = torch.device("cuda")
    sc = torch.from_numpy(scores).to(dev)
    lens_t = torch.tensor(lens, dtype=torch.int32, device=dev)
    ws = fasa.alloc_workspace(shape, max_t)
    # First call on a workspace full of one garbage byte (the select must fall back
    # to its full-row path and still be exact), then a call on the workspace the
    # select left behind (the fast path), then one on seeded random bytes (counts
    # and thresholds that look plausible but are wrong), then the fast path again.
    ws.fill_(0xA5)
    noise = torch.randint(0, 256, ws.shape, dtype=torch.uint8,
                          generator=torch.Generator().manual_seed(max_t + budget)).to(dev)
    for attempt in range(4):
        if attempt == 2:
            ws.copy_(noise)
        sel = torch.full((batch, H, max(cap, 1)), -7, dtype=torch.int32, device=dev)
        cnt = torch.full((batch, H), -7, dtype=torch.int32, device=dev)
        fasa.fasa_topk(shape, sc, lens_t, max_t, sel, cnt, ws)
        torch.cuda.synchronize()
        sel_h, cnt_h = sel.cpu().numpy(), cnt.cpu().numpy()
        for b in range(batch):
            for g in range(H):
                t = lens[b]
                ref, _ = O.select(scores[b, g, :t].astype(np.float64), budget, ns, nr)
                n = int(cnt_h[b, g])
                assert n == len(ref), (attempt, b, g, n, len(ref))
                np.testing.assert_array_equal(sel_h[b, g, :n], ref, err_msg=f"{case} b={b} g={g} call {attempt}")
                assert (sel_h[b, g, n:cap] == -1).all()


# ------------------------------------------------------------------------ FAC
@pytest.mark.parametrize("name", list(SMALL))
def test_fac_on_oracle_selection(name):
    say(f"[fac] {name}")
    inp, L = layer_for(name)
    cfg = inp.cfg
    units = oracle_units(inp)
    sel = np.full((cfg.batch, cfg.n_kv_heads, max(L.cap, 1)), -1, dtype=np.int32)
    cnt = np.zeros((cfg.batch, cfg.n_kv_heads), dtype=np.int32)
    for (b, g), (_, _, _, r) in units.items():
        cnt[b, g] = len(r["sel"])
        sel[b, g, :len(r["sel"])] = r["sel"]
    L.sel_idx.copy_(torch.from_numpy(sel))
    L.sel_count.copy_(torch.from_numpy(cnt))
    L.out.fill_(float("nan"))
    L.fac()
    torch.cuda.synchronize()
    out = L.out.cpu().numpy()
    G = cfg.group
    for (b, g), (q, K, V, r) in units.items():
        err = np.abs(out[b, g * G:(g + 1) * G] - r["out"]).max()
        assert err <= PR.OUT_ATOL[cfg.dtype], f"{name} b={b} g={g}: {err:.3e}"


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_fac_skips_entries_outside_the_cache(dtype):
    """fasa_fac over long, ragged selections with entries outside the cache mixed in.

    Entries of sel_idx[0..sel_count) below 0 or past the block table's last slot
    contribute nothing; the result is the oracle's FAC over the remaining rows (0
    for a unit with none).  With 32 units of about 9000 rows the bf16 launch gives
    each wave 144 rows, more than the 128 from which the matrix-core waves take
    the pipelined loop (row offsets resolved up front, next block in flight); the
    fp32 launch runs the vector waves."""
    say(f"[fac-skip] {dtype}")
    cfg = C["c2"].replace(dtype=dtype, batch=4, t=9000, budget=9000)
    inp = synth.make_inputs(cfg, seed=5, device="cpu")
    L = DeviceLayer(inp, device="cuda", with_slab=False)
    t = int(inp.seq_lens[0])
    lim = inp.max_blocks * 256
    rng = np.random.default_rng(11)
    sel = np.full((cfg.batch, cfg.n_kv_heads, L.cap), -1, dtype=np.int32)
    cnt = np.zeros((cfg.batch, cfg.n_kv_heads), dtype=np.int32)
    valid = {}
    for b in range(cfg.batch):
        for g in range(cfg.n_kv_heads):
            if (b, g) == (1, 7):
                valid[(b, g)] = np.zeros(0, dtype=np.int64)      # empty selection
                continue
            if (b, g) == (1, 6):
                row = np.array([-1, lim, -100, lim + 77, 2**31 - 1] * 20, dtype=np.int64)
                valid[(b, g)] = np.zeros(0, dtype=np.int64)      # nothing valid
            else:
                n = int(rng.integers(7000, L.cap + 1))
                keep = np.sort(rng.choice(t, size=n, replace=False))
                row = keep.copy()
                bad = rng.choice(n, size=n // 50, replace=False)
                row[bad] = rng.choice([-1, -100, lim, lim + 77, 2**31 - 1], size=len(bad))
                valid[(b, g)] = np.delete(keep, bad)
            cnt[b, g] = len(row)
            sel[b, g, :len(row)] = row
    L.sel_idx.copy_(torch.from_numpy(sel))
    L.sel_count.copy_(torch.from_numpy(cnt))
    L.out.fill_(float("nan"))
    L.fac()
    torch.cuda.synchronize()
    out = L.out.cpu().numpy()
    G = cfg.group
    for (b, g), rows in valid.items():
        got = out[b, g * G:(g + 1) * G]
        if len(rows) == 0:
            assert (got == 0).all(), f"{dtype} b={b} g={g}: no valid row, output not zero"
            continue
        q = inp.q[b, g * G:(g + 1) * G].double().cpu().numpy()
        K = unit_rows(inp, b, g, inp.k_pool).double().cpu().numpy()
        V = unit_rows(inp, b, g, inp.v_pool).double().cpu().numpy()
        ref, _ = O.fac(q, K[rows], V[rows], 1 / np.sqrt(128))
        err = np.abs(got - ref).max()
        assert err <= PR.OUT_ATOL[dtype], f"{dtype} b={b} g={g}: {err:.3e}"


# ------------------------------------------------------------------------ whole step
def _check_decode(inp, L, units, label, m=False):
    """Selections and outputs of the last fasa_decode (m: fasa_m_decode) on L."""
    torch.cuda.synchronize()
    return _check_arrays(inp, L, L.m_out if m else L.out, L.m_sel_idx if m else L.sel_idx,
                         L.m_sel_count if m else L.sel_count, units, label)


def _check_arrays(inp, L, out, sel, cnt, units, label):
    cfg = inp.cfg
    out, sel, cnt = out.cpu().numpy(), sel.cpu().numpy(), cnt.cpu().numpy()
    G = cfg.group
    same = 0
    for (b, g), (q, K, V, r) in units.items():
        t = int(inp.seq_lens[b])
        gs = sel[b, g, :cnt[b, g]].astype(np.int64)
        assert (sel[b, g, cnt[b, g]:L.cap] == -1).all()
        ok = PR.check_selection(gs, r, t, cfg.n_sink, cfg.n_recent, f"{label} b={b} g={g}")
        same += ok
        PR.check_output(out[b, g * G:(g + 1) * G], q, K, V, gs, r, ok, cfg.dtype,
                        1 / np.sqrt(128), f"{label} b={b} g={g}")
    return same


@pytest.mark.parametrize("name", list(SMALL))
def test_decode_end_to_end(name):
    say(f"[decode] {name}")
    inp, L = layer_for(name)
    L.out.fill_(float("nan"))
    L.decode()
    _check_decode(inp, L, oracle_units(inp), name)


@pytest.mark.parametrize("name", ["c4-ragged", "c3-shape", "wide-g4"])
def test_decode_with_garbage_workspace_is_identical(name):
    """The workspace carries a histogram between calls; garbage there may only
    cost speed, never change a result (the two-launch path with per-chunk
    candidates, the split path of large budgets, and the three-launch path)."""
    say(f"[decode garbage ws] {name}")
    inp, L = layer_for(name)
    L.decode()
    a = (L.out.clone(), L.sel_idx.clone(), L.sel_count.clone())
    noise = torch.randint(0, 256, L.workspace.shape, dtype=torch.uint8,
                          generator=torch.Generator().manual_seed(17)).to(L.workspace.device)
    for fill in ("byte", "random"):
        if fill == "byte":
            L.workspace.fill_(0x5A)
        else:
            L.workspace.copy_(noise)
        L.decode()
        b = (L.out.clone(), L.sel_idx.clone(), L.sel_count.clone())
        L.decode()
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert torch.equal(x, y), fill
        assert torch.equal(a[0], L.out) and torch.equal(a[1], L.sel_idx), fill


@pytest.mark.parametrize("name", ["c2-ragged", "c3-shape", "wide-g4", "fp32-gqa4"])
def test_decode_in_two_stages_is_identical(name):
    """fasa_decode_tip then fasa_decode_rest give fasa_decode's results bit for
    bit (the per-chunk-candidate path, the split path of large budgets, the
    three-launch path, an fp32 cache); so does a second TIP stage issued before
    the rest, as a loop timing the TIP stage alone leaves the workspace."""
    say(f"[two stages] {name}")
    inp, L = layer_for(name)
    L.decode()
    torch.cuda.synchronize()
    ref = (L.out.clone(), L.sel_idx.clone(), L.sel_count.clone())
    for tips in (1, 2):
        L.out.fill_(float("nan"))
        L.sel_idx.fill_(-7)
        L.sel_count.fill_(-7)
        for _ in range(tips):
            L.decode_tip()
        L.decode_rest()
        torch.cuda.synchronize()
        for x, y in zip(ref, (L.out, L.sel_idx, L.sel_count)):
            assert torch.equal(x, y), (name, tips)


def test_decode_without_slab_is_identical():
    name = "c2-ragged"
    say(f"[decode no-slab] {name}")
    inp, L = layer_for(name)
    L.decode(use_slab=True)
    a = (L.out.clone(), L.sel_idx.clone(), L.sel_count.clone())
    L.decode(use_slab=False)
    torch.cuda.synchronize()
    assert torch.equal(a[0], L.out) and torch.equal(a[1], L.sel_idx) and torch.equal(a[2], L.sel_count)


def test_determinism():
    name = "c5-ragged"
    say(f"[determinism] {name}")
    inp, L = layer_for(name)
    L.decode()
    a = (L.out.clone(), L.sel_idx.clone())
    for _ in range(3):
        L.decode()
    torch.cuda.synchronize()
    assert torch.equal(a[0], L.out) and torch.equal(a[1], L.sel_idx)


def test_all_fcs_and_full_budget_is_dense_attention():
    """With every FC dominant and B >= t the step is full attention (library SDPA in fp64)."""
    cfg = C["c2"].replace(n_fc=64, budget=100000, batch=2, t=None, t_range=(500, 1500))
    say("[dense special case]")
    inp = synth.make_inputs(cfg, seed=5)
    L = DeviceLayer(inp)
    L.decode()
    torch.cuda.synchronize()
    out = L.out.cpu().numpy()
    G = cfg.group
    for b in range(cfg.batch):
        t = int(inp.seq_lens[b])
        assert (L.sel_count[b].cpu().numpy() == t).all()
        for g in range(cfg.n_kv_heads):
            q = inp.q[b, g * G:(g + 1) * G].double()
            K = synth.unit_rows(inp, b, g, inp.k_pool).double()
            V = synth.unit_rows(inp, b, g, inp.v_pool).double()
            ref = torch.nn.functional.scaled_dot_product_attention(
                q[None, :, None, :], K[None, None].expand(1, G, t, 128),
                V[None, None].expand(1, G, t, 128))[0, :, 0, :].numpy()
            assert np.abs(out[b, g * G:(g + 1) * G] - ref).max() <= 2e-3


# ------------------------------------------------------------------------ dense decode
def _dense_ref(inp, b, g):
    """The oracle's dense decode of one unit: its rows copied into a one-head
    pool in logical order, read through an identity block table."""
    G = inp.cfg.group
    q = inp.q[b, g * G:(g + 1) * G].double().cpu().numpy()[None]
    K = unit_rows(inp, b, g, inp.k_pool).double().cpu().numpy()
    V = unit_rows(inp, b, g, inp.v_pool).double().cpu().numpy()
    t = K.shape[0]
    nblk = max((t + 255) // 256, 1)
    kp = np.zeros((nblk * 256, 128))
    vp = np.zeros((nblk * 256, 128))
    kp[:t], vp[:t] = K, V
    table = np.arange(nblk, dtype=np.int32)[None]
    return O.dense_decode(q, kp.reshape(nblk, 1, 256, 128), vp.reshape(nblk, 1, 256, 128), table,
                          np.array([t]))[(0, 0)]


def _check_dense(inp, L, units, label):
    """fasa_dense_decode against the oracle's full attention, unit by unit."""
    cfg = inp.cfg
    torch.cuda.synchronize()
    out = L.dense_out.cpu().numpy()
    G = cfg.group
    for b, g in sorted(units):
        err = np.abs(out[b, g * G:(g + 1) * G] - _dense_ref(inp, b, g)).max()
        assert err <= PR.OUT_ATOL[cfg.dtype], f"{label} b={b} g={g}: {err:.3e}"


@pytest.mark.parametrize("name", list(SMALL))
def test_dense_decode(name):
    say(f"[dense] {name}")
    inp, L = layer_for(name)
    L.dense()
    L.dense_out.fill_(float("nan"))
    L.dense()
    units = [(b, g) for b in range(inp.cfg.batch) for g in range(inp.cfg.n_kv_heads)]
    if len(units) > 64:
        units = units[::len(units) // 48]
    _check_dense(inp, L, units, name)


def test_dense_decode_edge_lengths():
    """t = 0 gives zeros; 1, 255, 256, 257 tokens cross the block edges."""
    cfg = C["c5"].replace(batch=6)
    say("[dense edge lengths]")
    inp = synth.make_inputs(cfg, seed=11, seq_lens=[0, 1, 255, 256, 257, 1100])
    L = DeviceLayer(inp, with_slab=False)
    L.dense()
    torch.cuda.synchronize()
    assert (L.dense_out[0] == 0).all()
    _check_dense(inp, L, [(b, g) for b in range(1, 6) for g in range(cfg.n_kv_heads)], "dense edge")


# ------------------------------------------------------------------------ FASA-M
M_CASES = ["c1", "c2-ragged", "c5-ragged", "fp32-gqa4", "g16-f5", "g2-f1-sink", "f32-fc32"]


@pytest.mark.parametrize("name", M_CASES)
def test_m_offload_bit_exact(name):
    """The host arrays hold exactly the non-dominant key columns (ascending,
    zero-padded) and the value rows of every cached token."""
    say(f"[fasa-m offload] {name}")
    inp, L = layer_for(name)
    L.m_setup()
    torch.cuda.synchronize()
    cfg = inp.cfg
    nd_n = 128 - 2 * cfg.n_fc
    for b in range(cfg.batch):
        t = int(inp.seq_lens[b])
        n = (t + 255) // 256
        blocks = torch.as_tensor(inp.block_table[b, :n].astype(np.int64))
        for g in range(cfg.n_kv_heads):
            K = unit_rows(inp, b, g, inp.k_pool)
            V = unit_rows(inp, b, g, inp.v_pool)
            got = L.m_knd[blocks, g].reshape(n * 256, -1)[:t]
            np.testing.assert_array_equal(got[:, :nd_n].float().numpy(),
                                          O.nondominant_rows(K.float().numpy(), inp.fc_idx[g]),
                                          err_msg=f"{name} b={b} g={g}")
            assert (got[:, nd_n:].float() == 0).all()
            assert torch.equal(L.m_v[blocks, g].reshape(n * 256, -1)[:t], V), f"{name} b={b} g={g}"


@pytest.mark.parametrize("name", M_CASES)
def test_m_decode(name):
    """FASA-M decode against the oracle, and its selection against fasa_decode's."""
    say(f"[fasa-m decode] {name}")
    inp, L = layer_for(name)
    L.m_setup()
    L.m_out.fill_(float("nan"))
    L.m_decode()
    L.decode()
    torch.cuda.synchronize()
    assert torch.equal(L.m_sel_count, L.sel_count)
    cap = L.cap
    assert torch.equal(L.m_sel_idx[..., :cap], L.sel_idx[..., :cap])
    _check_decode(inp, L, oracle_units(inp), name + " fasa-m", m=True)


@pytest.mark.parametrize("mode", ["resident", "prefetch"])
@pytest.mark.parametrize("name", ["c2-ragged", "c5-ragged", "fp32-gqa4", "g2-f1-sink"])
def test_m_reuse_consecutive_steps(name, mode):
    """FASA-M over four consecutive steps whose query changes every step (each
    query 0.9 times the last plus fresh noise), the rows of the previous
    selection reused: left in the workspace by the previous step (resident), or
    -- with the whole workspace overwritten before every step -- brought back by
    fasa_m_prefetch on a second stream while the step selects (prefetch).
    Every step against the oracle, bit for bit against fasa_m_decode of the
    same query (on a workspace of its own), and the reused rows equal to the
    overlap of consecutive selections."""
    import dataclasses
    cfg = SMALL[name]
    say(f"[fasa-m reuse] {name} {mode}")
    inp = synth.make_inputs(cfg, seed=3, device="cuda")
    L = DeviceLayer(inp)
    L.m_setup()
    ref_ws = torch.zeros_like(L.m_ws)
    ref = (torch.zeros_like(L.m_out), torch.zeros_like(L.m_sel_idx), torch.zeros_like(L.m_sel_count))
    qs = synth.drifting_queries(L.q.clone(), 4, rho=0.9, seed=1)
    sels = [(torch.full_like(L.m_sel_idx, -7), torch.full_like(L.m_sel_count, -7)) for _ in range(2)]
    hits = torch.zeros_like(L.m_sel_count)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    total_hits = total_rows = 0
    for n, q in enumerate(qs):
        par = n % 2
        cur = sels[par]
        prev = sels[1 - par] if n > 0 else None
        hits.zero_()
        L.m_out.fill_(float("nan"))
        if mode == "prefetch":
            L.m_ws.fill_(0xFF)
        fork = torch.cuda.Event()
        fork.record(main)
        side.wait_event(fork)
        if prev is not None and mode == "prefetch":
            L.m_prefetch(prev[0], prev[1], par, stream=side)
        L.m_select(q=q, sel_idx=cur[0], sel_count=cur[1], stream=main)
        join = torch.cuda.Event()
        join.record(side)
        main.wait_event(join)
        if prev is not None:
            L.m_finish(prev[0], prev[1], par, q=q, sel_idx=cur[0], sel_count=cur[1], hits=hits, stream=main)
        else:
            L.m_finish(None, None, par, q=q, sel_idx=cur[0], sel_count=cur[1], stream=main)
        torch.cuda.synchronize()
        got = (L.m_out.clone(), cur[0].clone(), cur[1].clone())
        inp_n = dataclasses.replace(inp, q=q)
        _check_arrays(inp_n, L, *got, oracle_units(inp_n), f"{name} {mode} step {n}")
        fasa.fasa_m_decode(L.shape, q, L.slab, L.m_knd, L.m_v, L.block_table, L.seq_lens, L.max_t, L.fc_idx,
                           ref[0], ref[1], ref[2], ref_ws)
        torch.cuda.synchronize()
        assert torch.equal(ref[0], got[0]) and torch.equal(ref[2], got[2]), (name, mode, n)
        assert torch.equal(ref[1][..., :L.cap], got[1][..., :L.cap]), (name, mode, n)
        if prev is not None:
            h = hits.cpu().numpy()
            c_sel, c_cnt = got[1].cpu().numpy(), got[2].cpu().numpy()
            p_sel, p_cnt = prev[0].cpu().numpy(), prev[1].cpu().numpy()
            for b in range(cfg.batch):
                for g in range(cfg.n_kv_heads):
                    both = np.intersect1d(c_sel[b, g, :c_cnt[b, g]], p_sel[b, g, :p_cnt[b, g]])
                    assert h[b, g] == len(both), (name, n, b, g, h[b, g], len(both))
            total_hits += int(h.sum())
            total_rows += int(got[2].sum().item())
    say(f"  {total_hits} of {total_rows} rows of steps 1-3 reused")
    assert total_hits > 0


def test_m_decode_full_size_8b_layer():
    """FASA-M on the Llama-3-8B-shaped layer at t = 32768, every unit."""
    cfg = C["c2"]
    say(f"[fasa-m full] {cfg.name}")
    inp = synth.make_inputs(cfg, seed=0, device="cuda")
    L = DeviceLayer(inp)
    L.m_setup()
    L.m_decode()
    _check_decode(inp, L, oracle_units(inp), "c2 fasa-m", m=True)
    del L, inp
    torch.cuda.empty_cache()


# ------------------------------------------------------------------------ CA calibration
CA_CASES = ["c1", "c2-ragged", "c5-ragged", "fp32-gqa4", "g16-f5"]


def _ca_hits(L, k_top):
    """The kernel's hit counts and the 65 top-K lists of every unit behind them."""
    cfg = L.cfg
    ws = torch.zeros(fasa.fasa_ca_workspace_size(L.shape, L.max_t, k_top), dtype=torch.uint8, device="cuda")
    hits = torch.full((cfg.batch, cfg.n_kv_heads, 64), -1, dtype=torch.int32, device="cuda")
    cap = min(k_top, L.max_t)
    lists = torch.full((cfg.batch, cfg.n_kv_heads, 65, cap), -7, dtype=torch.int32, device="cuda")
    fasa.fasa_ca_hits(L.shape, L.q, L.k_pool, L.block_table, L.seq_lens, L.max_t, k_top, hits, ws, topk=lists)
    torch.cuda.synchronize()
    return hits, lists.cpu().numpy()


def _ca_check_unit(inp, lists, hits, b, g, k_top, where):
    """The unit's lists validated against the fp64 oracle, then its hits against
    the intersections of those lists.  Returns the number of lists in the band."""
    G = inp.cfg.group
    q = inp.q[b, g * G:(g + 1) * G].double().cpu().numpy()
    K = unit_rows(inp, b, g, inp.k_pool).double().cpu().numpy()
    expect, differ = PR.check_ca_lists(lists[b, g], q, K, k_top, where)
    np.testing.assert_array_equal(hits[b, g], expect, err_msg=where)
    if differ == 0:
        np.testing.assert_array_equal(hits[b, g], np.rint(O.contextual_agreement(q, K, k_top) * k_top),
                                      err_msg=where)
    return differ


@pytest.mark.parametrize("k_top", [64, 256])
@pytest.mark.parametrize("name", CA_CASES)
def test_ca_hits_exact(name, k_top):
    """The 65 top-K lists of every sampled unit against the fp64 oracle (tie
    band), and the hit counts bit-exact against those lists."""
    say(f"[ca hits] {name} K={k_top}")
    inp, L = layer_for(name)
    h, lists = _ca_hits(L, k_top)
    h = h.cpu().numpy()
    cfg = inp.cfg
    units = [(b, g) for b in range(cfg.batch) for g in range(cfg.n_kv_heads)]
    if len(units) > 12:
        units = units[::len(units) // 12]
    differ = sum(_ca_check_unit(inp, lists, h, b, g, k_top, f"{name} b={b} g={g}") for b, g in units)
    say(f"  {len(units)} units, {differ} of {65 * len(units)} lists differ inside the band")


def test_ca_calibration_sample_steps():
    """Eight steps of one calibration sample (block tables sharing one
    sequence's blocks, lengths 1990..1997), K = 256: every unit's lists and hits
    validated, then the dominant FCs of the summed hits against the oracle's
    ranking of the mean CA."""
    cfg = C["c2"].replace(batch=8, t=2000)
    say("[ca sample steps]")
    inp = synth.make_inputs(cfg, seed=13)
    inp.block_table[:] = inp.block_table[0]
    inp.seq_lens[:] = 1990 + np.arange(8, dtype=np.int32)
    L = DeviceLayer(inp, with_slab=False)
    k_top = 256
    hits, lists = _ca_hits(L, k_top)
    h = hits.cpu().numpy()
    for b in range(cfg.batch):
        for g in range(cfg.n_kv_heads):
            _ca_check_unit(inp, lists, h, b, g, k_top, f"sample b={b} g={g}")
    fc = torch.full((cfg.n_kv_heads, 16), -1, dtype=torch.int32, device="cuda")
    fasa.fasa_ca_dominant(L.shape, hits, cfg.batch, 16, fc)
    torch.cuda.synchronize()
    got = fc.cpu().numpy()
    for g in range(cfg.n_kv_heads):
        mean = h[:, g, :].sum(axis=0) / float(cfg.batch * k_top)
        assert list(got[g]) == list(O.dominant_fcs(mean, 16)), g
    fasa.fasa_check_fc_idx(L.shape, got)     # a valid fc_idx for the decode path


def test_empty_and_tiny_sequences():
    cfg = C["c5"].replace(batch=5, budget=16, n_sink=4, n_recent=8)
    say("[edge lengths]")
    inp = synth.make_inputs(cfg, seed=9, seq_lens=[0, 1, 13, 29, 300])
    L = DeviceLayer(inp)
    L.out.fill_(float("nan"))
    L.decode()
    torch.cuda.synchronize()
    assert (L.out[0] == 0).all()
    assert (L.sel_count[0] == 0).all()
    _check_decode(inp, L, {k: v for k, v in oracle_units(inp).items() if k[0] > 0}, "edge")


def test_decode_long_rows_ragged():
    """The Qwen2.5-7B-shaped layer (groups of 7, B = 1024) on the
    histogram-filtered list path (TIP's per-chunk lists together too long for
    the selecting workgroup, cut down with the unit histogram), with one-head
    selecting workgroups over 1024-row lists: a 90000-token row, a short one
    just past the budget, an empty sequence and a one-token one."""
    cfg = C["c4"].replace(batch=4)
    say("[long rows] c4 shape, lengths 90000 1500 0 1")
    inp = synth.make_inputs(cfg, seed=21, seq_lens=[90000, 1500, 0, 1])
    L = DeviceLayer(inp)
    assert fasa.fasa_decode_path(L.shape, L.max_t) == fasa.PATH_FILTERED_LISTS
    L.out.fill_(float("nan"))
    L.decode()
    torch.cuda.synchronize()
    assert (L.out[2] == 0).all() and (L.sel_count[2] == 0).all()
    _check_decode(inp, L, {k: v for k, v in oracle_units(inp).items() if k[0] != 2}, "long rows")


def _score_bins(S: np.ndarray) -> np.ndarray:
    """Coarse bins (top 11 bits) of the order-preserving 32-bit images of fp32
    scores, -0.0 taken as +0.0 -- the histogram's definition."""
    u = np.ascontiguousarray(S, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = np.where(u == 0x80000000, 0, u)
    key = np.where(u & 0x80000000, (~u) & 0xFFFFFFFF, u | 0x80000000)
    return (key >> 21).astype(np.int64)


def test_decode_filtered_lists_fallbacks():
    """The histogram-filtered list path at 128 chunks per row (Qwen2.5-7B
    layer, B = 1024, rows of 131072 and 70001 tokens), with both ways a unit's
    lists can fail it planted: in unit (0, 0) chunk 5 holds 200 copies of one
    high key (its list outgrows what the selecting workgroup reads of a list),
    in unit (1, 1) the top-B sits in one chunk (a chunk that left keys out has
    its threshold above the B-th key's bin).  TIP's unit histograms (the
    filter's threshold) must equal the bin counts of its scores; every unit
    must match the oracle; a workspace of random bytes (a wrong histogram and
    arrival counters) must give the same result."""
    cfg = C["c4"].replace(batch=2)
    say("[filtered lists] c4 shape, lengths 131072 70001, long list + clustered")
    inp = synth.make_inputs(cfg, seed=53, seq_lens=[131072, 70001])
    G = cfg.group
    # Unit (0, 0): 200 copies of chunk 5's best key inside chunk 5.
    q = inp.q[0, 0:G].double().numpy()
    K = unit_rows(inp, 0, 0, inp.k_pool).double().numpy()
    S = O.tip_scores(q, K, inp.fc_idx[0])
    src = 5 * 1024 + int(np.argmax(S[5 * 1024:6 * 1024]))
    row = inp.k_pool[int(inp.block_table[0, src // 256]), 0, src % 256].clone()
    pos = [j for j in range(5 * 1024, 6 * 1024, 5) if j != src][:200]
    for j in pos:
        inp.k_pool[int(inp.block_table[0, j // 256]), 0, j % 256] = row
    # Unit (1, 1): keys of 40000 .. 41023 pushed along the folded dominant query.
    qf = inp.q[1, G:2 * G].float().sum(0)
    u = torch.zeros(128)
    for i in inp.fc_idx[1]:
        u[2 * i:2 * i + 2] = qf[2 * i:2 * i + 2]
    u = u / u.norm()
    for j in range(40000, 41024):
        p, s_ = int(inp.block_table[1, j // 256]), j % 256
        inp.k_pool[p, 1, s_] = (inp.k_pool[p, 1, s_].float() + (40.0 + 0.01 * j) * u).to(inp.k_pool.dtype)
    L = DeviceLayer(inp)
    assert fasa.fasa_decode_path(L.shape, L.max_t) == fasa.PATH_FILTERED_LISTS
    L.workspace.zero_()
    L.decode_tip()
    L.tip()
    torch.cuda.synchronize()
    units = cfg.batch * cfg.n_kv_heads
    hist = L.workspace[:units * 2048 * 4].view(torch.int32).reshape(cfg.batch, cfg.n_kv_heads, 2048).cpu().numpy()
    Sg = L.scores.cpu().numpy()
    for b in range(cfg.batch):
        t = int(inp.seq_lens[b])
        c_lo = min(cfg.n_sink, t)
        c_hi = max(c_lo, t - cfg.n_recent)
        for g in range(cfg.n_kv_heads):
            want = np.bincount(_score_bins(Sg[b, g, c_lo:c_hi]), minlength=2048)
            np.testing.assert_array_equal(hist[b, g], want, err_msg=f"b={b} g={g}")
    L.out.fill_(float("nan"))
    L.decode()
    torch.cuda.synchronize()
    units_o = oracle_units(inp)
    _check_decode(inp, L, units_o, "filtered lists")
    sel = units_o[(1, 1)][3]["sel"]
    assert ((sel >= 40000) & (sel < 41024)).all(), "the construction failed to cluster the top-B"
    a = (L.out.clone(), L.sel_idx.clone(), L.sel_count.clone())
    L.workspace.copy_(torch.randint(0, 256, L.workspace.shape, dtype=torch.uint8,
                                    generator=torch.Generator().manual_seed(53)).to(L.workspace.device))
    for _ in range(2):
        L.decode()
        torch.cuda.synchronize()
        for x, y in zip(a, (L.out, L.sel_idx, L.sel_count)):
            assert torch.equal(x, y), "random workspace"


def test_decode_filtered_lists_fp32_forced():
    """The histogram-filtered list path with fp32 caches (fp64 softmax and
    weighted sum, the unmasked row batches included) and forced sink and
    recent tokens: the Qwen2.5-7B layer shape at rows of 131072 and 77777
    tokens, B = 1024 plus 4 + 64 forced; every unit against the oracle."""
    cfg = C["c4"].replace(dtype="fp32", batch=2, n_sink=4, n_recent=64)
    say("[filtered lists fp32] c4 shape fp32, lengths 131072 77777, 4 + 64 forced")
    inp = synth.make_inputs(cfg, seed=57, seq_lens=[131072, 77777])
    L = DeviceLayer(inp)
    assert fasa.fasa_decode_path(L.shape, L.max_t) == fasa.PATH_FILTERED_LISTS
    L.out.fill_(float("nan"))
    L.decode()
    torch.cuda.synchronize()
    _check_decode(inp, L, oracle_units(inp), "filtered lists fp32")


def test_decode_filtered_lists_bf16_forced():
    """The histogram-filtered list path with bf16 caches and forced tokens
    (3 sink, 37 recent): lists of B + 40 rows end in a part batch, and a
    900-token row keeps every token (a list of 900 rows), so the 8-lanes-per-row
    FAC runs its masked batches as well as the unmasked ones.  Qwen2.5-7B layer
    shape, rows of 131072, 77777 and 900 tokens; every unit against the oracle."""
    cfg = C["c4"].replace(batch=3, n_sink=3, n_recent=37)
    say("[filtered lists bf16] c4 shape, lengths 131072 77777 900, 3 + 37 forced")
    inp = synth.make_inputs(cfg, seed=59, seq_lens=[131072, 77777, 900])
    L = DeviceLayer(inp)
    assert fasa.fasa_decode_path(L.shape, L.max_t) == fasa.PATH_FILTERED_LISTS
    L.out.fill_(float("nan"))
    L.decode()
    torch.cuda.synchronize()
    _check_decode(inp, L, oracle_units(inp), "filtered lists bf16 forced")


@pytest.mark.parametrize("kind", ["lists", "filtered"])
def test_decode_lists_whole_v_rows(kind):
    """TIP's lists with more query heads than CUs to split V over (bf16, one
    head per workgroup, 2 x heads > 256 CUs): each head keeps one workgroup
    over whole V rows.  The 8B-layer shape at batch 20 (640 heads, rows of
    1500-3000 tokens: whole lists) and the Qwen2.5-7B shape at batch 10 (280
    heads, rows of 90000-100000 tokens: filtered lists); every unit against
    the oracle."""
    if kind == "lists":
        cfg = C["c2"].replace(batch=20, t=None, t_range=(1500, 3000))
        want = fasa.PATH_LISTS
    else:
        cfg = C["c4"].replace(batch=10, t=None, t_range=(90000, 100000))
        want = fasa.PATH_FILTERED_LISTS
    say(f"[lists whole V] {kind}: {cfg.name} batch {cfg.batch}")
    inp = synth.make_inputs(cfg, seed=67)
    L = DeviceLayer(inp)
    assert fasa.fasa_decode_path(L.shape, L.max_t) == want
    L.out.fill_(float("nan"))
    L.decode()
    torch.cuda.synchronize()
    _check_decode(inp, L, oracle_units(inp), f"lists whole V {kind}")


def test_decode_filtered_lists_in_two_stages():
    """The histogram-filtered list path (Qwen2.5-7B layer, B = 1024, a ragged
    batch of three rows up to 131072 tokens) split into fasa_decode_tip and
    fasa_decode_rest gives fasa_decode's results bit for bit; so does a second
    TIP stage before the rest, which leaves every unit histogram at twice its
    counts (a threshold bin that keeps fewer than B keys, so the select takes
    its slower route), and a decode that follows it on the same workspace."""
    cfg = C["c4"].replace(batch=3, t=None, t_range=(40000, 131072))
    say("[filtered lists two stages] c4 shape, 3 ragged rows")
    inp = synth.make_inputs(cfg, seed=61)
    L = DeviceLayer(inp)
    assert fasa.fasa_decode_path(L.shape, L.max_t) == fasa.PATH_FILTERED_LISTS
    L.decode()
    torch.cuda.synchronize()
    ref = (L.out.clone(), L.sel_idx.clone(), L.sel_count.clone())
    assert not torch.isnan(ref[0]).any()
    for tips in (1, 2, 1):
        L.out.fill_(float("nan"))
        L.sel_idx.fill_(-7)
        L.sel_count.fill_(-7)
        for _ in range(tips):
            L.decode_tip()
        L.decode_rest()
        torch.cuda.synchronize()
        for x, y in zip(ref, (L.out, L.sel_idx, L.sel_count)):
            assert torch.equal(x, y), tips
    L.decode()
    torch.cuda.synchronize()
    for x, y in zip(ref, (L.out, L.sel_idx, L.sel_count)):
        assert torch.equal(x, y), "decode after the stages"


def test_decode_tip_histograms_ragged():
    """A ragged batch of 64 sequences x 8 kv heads (512 units, rows up to 16384
    tokens, B = 512 plus 4 + 64 forced: the three-launch step, TIP building the
    unit histograms).  Lengths at chunk edges, odd chunk counts, 0 and 1.  The
    histograms only steer the select's speed, so a wrong one would pass every
    parity test: the per-unit histograms TIP leaves in a zeroed workspace must
    equal the bin counts of the same TIP scores.  Then every unit's step against
    the oracle."""
    lens = [16384, 0, 1, 1023, 1024, 1025, 5 * 1024, 5 * 1024 + 1, 7 * 1024 - 1, 9000, 12345, 16000, 67, 68, 69]
    rng = np.random.default_rng(31)
    lens += [int(x) for x in rng.integers(100, 16385, size=64 - len(lens))]
    cfg = C["c5"].replace(batch=64)
    say("[tip histograms] ragged 64 x 8, t <= 16384")
    inp = synth.make_inputs(cfg, seed=31, seq_lens=lens, device="cuda")
    L = DeviceLayer(inp)
    L.workspace.zero_()
    L.decode_tip()
    L.tip()
    torch.cuda.synchronize()
    units = cfg.batch * cfg.n_kv_heads
    hist = L.workspace[:units * 2048 * 4].view(torch.int32).reshape(cfg.batch, cfg.n_kv_heads, 2048).cpu().numpy()
    S = L.scores.cpu().numpy()
    for b in range(cfg.batch):
        t = int(inp.seq_lens[b])
        c_lo = min(cfg.n_sink, t)
        c_hi = max(c_lo, t - cfg.n_recent)
        for g in range(cfg.n_kv_heads):
            want = np.bincount(_score_bins(S[b, g, c_lo:c_hi]), minlength=2048)
            np.testing.assert_array_equal(hist[b, g], want, err_msg=f"b={b} g={g} t={t}")
    L.out.fill_(float("nan"))
    L.decode()
    torch.cuda.synchronize()
    assert (L.out[1] == 0).all() and (L.sel_count[1] == 0).all()
    _check_decode(inp, L, {k: v for k, v in oracle_units(inp).items() if k[0] != 1}, "tip histograms")


def test_graph_capture_replays():
    name = "c2-ragged"
    say(f"[graph] {name}")
    inp, L = layer_for(name)
    L.decode()
    torch.cuda.synchronize()
    ref = (L.out.clone(), L.sel_idx.clone())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        L.out.zero_()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            L.decode()
    torch.cuda.current_stream().wait_stream(s)
    for i in range(3):
        L.out.fill_(float("nan"))
        L.sel_idx.fill_(-5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(L.out, ref[0]) and torch.equal(L.sel_idx, ref[1]), f"replay {i}"


# ------------------------------------------------------------------------ full sizes
# Units the oracle checks at full size: every unit of c1-c4; for the ragged
# batch every kv head of its shortest, median and longest sequence.
FULL_SAMPLES = {
    "c5": "extremes",
}


@pytest.mark.parametrize("kind", ["lists", "filtered"])
def test_decode_duplicate_keys_tie_to_lower_index(kind):
    """Exact score ties through the whole decode step: in every unit, 30 copies
    of the key of the token the oracle ranks B - 10 are written at other
    positions (in its own 1024-token chunk and in others, before and after it),
    so the B-th score is shared by many tokens.  TIP gives identical rows
    bit-identical scores, and the select must keep the lowest indices among
    them, exactly as the oracle's (-S, j) order does.  Through TIP's lists (8B
    layer shape, rows of 6000-9000 tokens) and through the lists filtered by the
    unit histogram (Qwen2.5-7B layer shape, rows of 90000-100000 tokens)."""
    if kind == "lists":
        cfg = C["c2"].replace(batch=2, n_q_heads=8, n_kv_heads=2, t=None, t_range=(6000, 9000), budget=200)
        want_path = fasa.PATH_LISTS
    else:
        cfg = C["c4"].replace(batch=2, t=None, t_range=(90000, 100000))
        want_path = fasa.PATH_FILTERED_LISTS
    say(f"[decode duplicate keys] {kind}")
    inp = synth.make_inputs(cfg, seed=41)
    rng = np.random.default_rng(41)
    G = cfg.group
    dup = {}
    for b in range(cfg.batch):
        t = int(inp.seq_lens[b])
        for g in range(cfg.n_kv_heads):
            q = inp.q[b, g * G:(g + 1) * G].double().numpy()
            K = unit_rows(inp, b, g, inp.k_pool).double().numpy()
            S = O.tip_scores(q, K, inp.fc_idx[g])
            order = np.lexsort((np.arange(t), -S))
            src = int(order[cfg.budget - 10])
            near = rng.choice(np.arange(max(0, src - 900), min(t, src + 900)), size=10, replace=False)
            far = rng.choice(t, size=20, replace=False)
            pos = np.setdiff1d(np.concatenate([near, far]), order[:cfg.budget - 10])
            pos = pos[pos != src]
            row = inp.k_pool[int(inp.block_table[b, src // 256]), g, src % 256].clone()
            for j in pos:
                inp.k_pool[int(inp.block_table[b, j // 256]), g, int(j) % 256] = row
            dup[(b, g)] = np.sort(np.append(pos, src))
    L = DeviceLayer(inp)
    assert fasa.fasa_decode_path(L.shape, L.max_t) == want_path
    L.out.fill_(float("nan"))
    L.decode()
    units = oracle_units(inp)
    _check_decode(inp, L, units, "duplicate keys")
    for (b, g), grp in dup.items():
        got = np.intersect1d(L.selection(b, g), grp)
        want = np.intersect1d(units[(b, g)][3]["sel"], grp)
        assert 0 < len(want) < len(grp), (b, g, len(want), len(grp))   # the B-th score is shared
        np.testing.assert_array_equal(got, want, err_msg=f"b={b} g={g}: tied copies kept")


def test_decode_clustered_top_scores():
    """Every unit's top-B inside one 1024-token chunk (keys there pushed along
    the folded dominant query): a chunk's candidate list then cannot cover the
    top-B, and the select must notice and still return the exact set."""
    cfg = C["c2"].replace(batch=2, n_q_heads=8, n_kv_heads=2, t=None, t_range=(8000, 12000), budget=256)
    say("[decode clustered]")
    inp = synth.make_inputs(cfg, seed=43)
    G = cfg.group
    for b in range(cfg.batch):
        for g in range(cfg.n_kv_heads):
            qf = inp.q[b, g * G:(g + 1) * G].float().sum(0)
            u = torch.zeros(128)
            for i in inp.fc_idx[g]:
                u[2 * i:2 * i + 2] = qf[2 * i:2 * i + 2]
            u = u / u.norm()
            for j in range(3072 + 64 * g, 4096):
                p, s_ = int(inp.block_table[b, j // 256]), j % 256
                k = inp.k_pool[p, g, s_].float() + (40.0 + 0.01 * j) * u
                inp.k_pool[p, g, s_] = k.to(inp.k_pool.dtype)
    L = DeviceLayer(inp)
    L.out.fill_(float("nan"))
    L.decode()
    units = oracle_units(inp)
    _check_decode(inp, L, units, "clustered")
    for (b, g), (_, _, _, r) in units.items():
        assert ((r["sel"] >= 3072) & (r["sel"] < 4096)).all(), "the construction failed to cluster the top-B"


@pytest.mark.parametrize("budget", [512, 1500])
def test_decode_ragged_many_chunks(budget):
    """Nine sequences x 8 kv heads, max_t 65536, lengths at chunk edges, 0 and
    at most n_sink + n_recent, every unit against the oracle.  B = 512 takes
    the two-launch step (TIP's candidate lists); B = 1500 the filter launch,
    whose grid (32 x 8 x 9 workgroups) reads each sequence's length before its
    scores, then the select launch and the split FAC."""
    cfg = C["c5"].replace(batch=9, budget=budget)
    say(f"[decode ragged many chunks] B={budget}")
    lens = [65536, 100, 2047, 2048, 2049, 30000, 1023, 0, 65000]
    inp = synth.make_inputs(cfg, seed=47, seq_lens=lens)
    L = DeviceLayer(inp)
    L.out.fill_(float("nan"))
    L.decode()
    torch.cuda.synchronize()
    assert (L.out[7] == 0).all() and (L.sel_count[7] == 0).all()
    _check_decode(inp, L, {k: v for k, v in oracle_units(inp).items() if k[0] != 7}, f"ragged B={budget}")


@pytest.mark.parametrize("name", ["c2-ragged", "fp32-gqa4", "c5-ragged", "c3-shape"])
def test_per_head_fc_counts(name):
    """Per-head N_tip: kv head g uses only the first F - (g mod F) of its FCs
    (the rest of its fc_idx row is -1); TIP, the select and FAC against the
    oracle on the same rows."""
    cfg = SMALL[name]
    say(f"[per-head n_fc] {name}")
    inp = synth.make_inputs(cfg, seed=29)
    F = cfg.n_fc
    for g in range(cfg.n_kv_heads):
        drop = g % F
        if drop:
            inp.fc_idx[g, F - drop:] = -1
    L = DeviceLayer(inp)
    fasa.fasa_check_fc_idx(L.shape, inp.fc_idx)
    L.out.fill_(float("nan"))
    L.decode()
    _check_decode(inp, L, oracle_units(inp), name + " per-head n_fc")


def test_per_layer_budgets_in_one_graph():
    """Per-layer budgets (PyramidKV-style): each layer's call carries its own
    shape, so layers with budgets 48, 300 and 1500 run back to back in one
    captured graph; every replay matches the oracle at each layer's budget."""
    say("[per-layer budgets]")
    layers = []
    for k, budget in enumerate((48, 300, 1500)):
        cfg = C["c2"].replace(batch=2, t=None, t_range=(2500, 4000), budget=budget)
        inp = synth.make_inputs(cfg, seed=31 + k)
        layers.append((inp, DeviceLayer(inp)))
    for _, L in layers:
        L.decode()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            for _, L in layers:
                L.decode()
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(2):
        for _, L in layers:
            L.out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for inp, L in layers:
            _check_decode(inp, L, oracle_units(inp), f"budget {inp.cfg.budget} replay {rep}")


@pytest.mark.parametrize("t", [524288, 524289 + 300])
def test_longest_contexts(t):
    """The selecting FAC keeps a sequence's block-table row in LDS, up to 2048
    blocks (524288 tokens); one token more takes the select-then-split path.
    Both sides of that boundary, every unit against the oracle."""
    cfg = C["c2"].replace(batch=1, n_q_heads=4, n_kv_heads=1, t=t)
    say(f"[longest] t={t}")
    inp = synth.make_inputs(cfg, seed=17, device="cuda")
    L = DeviceLayer(inp)
    L.decode()
    _check_decode(inp, L, oracle_units(inp), f"t={t}")
    L.dense()
    _check_dense(inp, L, [(0, 0)], f"t={t} dense")
    del L, inp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("key", ["c1", "c2", "c3", "c4", "c5"])
def test_full_size_configs(key):
    """The workloads at their full sizes, in the launch configuration the benchmark
    times; the oracle checks sampled (sequence, kv head) units."""
    cfg = C[key]
    say(f"[full] {key} {cfg.name}")
    inp = synth.make_inputs(cfg, seed=0, device="cuda")
    L = DeviceLayer(inp)
    L.decode()
    torch.cuda.synchronize()
    pick = FULL_SAMPLES.get(key)
    if pick == "extremes":
        order = np.argsort(inp.seq_lens)
        seqs = [int(order[0]), int(order[len(order) // 2]), int(order[-1])]
        pick = [(b, g) for b in seqs for g in range(cfg.n_kv_heads)]
    units = oracle_units(inp, set(pick) if pick else None)
    _check_decode(inp, L, units, key)
    say(f"[full dense] {key}")
    L.dense()
    dense_units = sorted(units)
    if len(dense_units) > 24:
        dense_units = dense_units[::len(dense_units) // 24]
    _check_dense(inp, L, dense_units, key + " dense")
    del L, inp
    torch.cuda.empty_cache()
