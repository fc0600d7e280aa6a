"""Seeded synthetic inputs for one FASA decode step.

This module produces the *inputs* of the decode hot path: post-RoPE query
vectors, a paged post-RoPE key cache and value cache, per-kv-head dominant
frequency-chunk (FC) indices, sequence lengths and block tables.  It holds none
of the method's arithmetic (no scoring, no selection, no attention): the fp64
oracle under ``oracle/`` and the HIP library both consume what it returns.

Workload shapes follow the decode layers the FASA pages evaluate (Llama-3-8B,
Qwen2.5-7B and Mistral-7B shaped heads with head_dim 128, 4K-128K contexts);
the data is synthetic because no model weights or datasets are used:

* pre-RoPE q, k, v ~ N(0, 1), fp32 draws;
* per kv head, 4 seeded "massive" channels scaled by 8 in k, v and in every
  query head of the group (long-context activations have a few outlier
  channels; the scale makes logits O(10));
* interleaved RoPE: FC i is the dimension pair (2i, 2i+1) with angular
  frequency theta_i = base^(-2i/d) (paper-graph-ui review of FASA, section 3.4,
  "RoPE from a Frequency-Chunk Perspective");
* keys sit at positions 0..t-1, the query at position t;
* the cache is paged in 256-token blocks whose physical order is a seeded
  permutation, so that paging is never contiguous;
* dominant FC indices are a seeded sorted uniform subset of [0, d/2) per kv
  head (the pages calibrate them on a model, which is not available here).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

import numpy as np
import torch

HEAD_DIM = 128
BLOCK = 256
N_MASSIVE = 4
MASSIVE_SCALE = 8.0
BASE_SEED = 20260203


@dataclasses.dataclass(frozen=True)
class Config:
    """One decode-layer workload."""

    key: str
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    t: Optional[int]                      # fixed context length, or None if ragged
    t_range: Optional[Tuple[int, int]]    # inclusive range of ragged lengths
    theta: float                          # RoPE base
    dtype: str                            # "fp32" | "bf16" (cache and query)
    n_fc: int                             # dominant FCs per kv head
    budget: int                           # B, tokens kept by the top-B select
    n_sink: int = 0                       # always-kept first tokens
    n_recent: int = 0                     # always-kept last tokens
    head_dim: int = HEAD_DIM
    index: int = 0                        # seeds differ per workload

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "fp32" else 2

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "c1": Config("c1", "tiny-1q1kv-t4096-fp32-B256", batch=1, n_q_heads=1, n_kv_heads=1,
                 t=4096, t_range=None, theta=1e4, dtype="fp32", n_fc=16, budget=256, index=1),
    "c2": Config("c2", "llama3-8b-layer-t32768-bf16-B256", batch=1, n_q_heads=32, n_kv_heads=8,
                 t=32768, t_range=None, theta=5e5, dtype="bf16", n_fc=16, budget=256, index=2),
    "c3": Config("c3", "llama3-8b-layer-batch16-t32768-bf16-B6193", batch=16, n_q_heads=32,
                 n_kv_heads=8, t=32768, t_range=None, theta=5e5, dtype="bf16", n_fc=16,
                 budget=6193, index=3),
    "c4": Config("c4", "qwen2.5-7b-layer-batch4-t131072-bf16-F8-B1024", batch=4, n_q_heads=28,
                 n_kv_heads=4, t=131072, t_range=None, theta=1e6, dtype="bf16", n_fc=8,
                 budget=1024, index=4),
    "c5": Config("c5", "mistral-7b-layer-ragged64-t4096..65536-paged-bf16-B512+4+64", batch=64,
                 n_q_heads=32, n_kv_heads=8, t=None, t_range=(4096, 65536), theta=1e6,
                 dtype="bf16", n_fc=16, budget=512, n_sink=4, n_recent=64, index=5),
}


@dataclasses.dataclass
class Inputs:
    """Everything one decode step consumes.  Tensors live on ``device``."""

    cfg: Config
    seed: int
    seq_lens: np.ndarray          # int32 [batch]
    fc_idx: np.ndarray            # int32 [H_kv][F], each row sorted, distinct, in [0, d/2)
    massive: np.ndarray           # int32 [H_kv][4] channel ids scaled by 8
    block_table: np.ndarray       # int32 [batch][max_blocks]; unused entries -> spare block
    n_blocks: int                 # physical blocks in the pool (last one is a spare)
    q: torch.Tensor               # [batch][H_q][d]   cfg dtype, post-RoPE at position t_b
    k_pool: torch.Tensor          # [n_blocks][H_kv][256][d] cfg dtype, post-RoPE
    v_pool: torch.Tensor          # [n_blocks][H_kv][256][d] cfg dtype

    @property
    def max_t(self) -> int:
        return int(self.seq_lens.max()) if len(self.seq_lens) else 0

    @property
    def max_blocks(self) -> int:
        return self.block_table.shape[1]


def rope_angles(positions: torch.Tensor, theta: float, head_dim: int) -> torch.Tensor:
    """fp64 angles m * theta_i for every position m and FC i: [len(positions)][d/2]."""
    i = torch.arange(head_dim // 2, dtype=torch.float64, device=positions.device)
    inv = theta ** (-2.0 * i / head_dim)
    return positions.to(torch.float64)[:, None] * inv[None, :]


def apply_rope(x: torch.Tensor, positions: torch.Tensor, theta: float) -> torch.Tensor:
    """Rotate every FC of ``x`` (shape [..., n, d]) by its position's angle.

    The rotation acts on the FC as a row vector times R_{m,theta_i} with
    R = [[cos, -sin], [sin, cos]], i.e.
        x'_{2i}   =  x_{2i} cos(m theta_i) + x_{2i+1} sin(m theta_i)
        x'_{2i+1} = -x_{2i} sin(m theta_i) + x_{2i+1} cos(m theta_i).
    With this direction the pages' relative form q^[i] R_{t1-t2} k^[i]^T of
    the FC-wise score equals the dot product of the rotated vectors exactly.
    Computed in fp64; the caller casts.
    """
    ang = rope_angles(positions, theta, x.shape[-1])            # [n][d/2]
    c, s = torch.cos(ang), torch.sin(ang)
    x = x.to(torch.float64)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    y = torch.empty_like(x)
    y[..., 0::2] = x0 * c + x1 * s
    y[..., 1::2] = -x0 * s + x1 * c
    return y


def _seeds(cfg: Config, seed: int):
    ss = np.random.SeedSequence([BASE_SEED + cfg.index, seed])
    kids = ss.spawn(7)   # fc_idx, massive, q, k, v, lengths, block permutation
    return kids


def draw_lengths(cfg: Config, seed: int = 0) -> np.ndarray:
    kids = _seeds(cfg, seed)
    if cfg.t is not None:
        return np.full(cfg.batch, cfg.t, dtype=np.int32)
    lo, hi = cfg.t_range
    rng = np.random.default_rng(kids[5])
    return rng.integers(lo, hi + 1, size=cfg.batch).astype(np.int32)


def make_inputs(cfg: Config, seed: int = 0, device="cpu", seq_lens=None,
                pad_value: float = float("nan")) -> Inputs:
    """Draw one decode step's inputs for ``cfg``.

    ``seq_lens`` overrides the drawn lengths (edge-case tests).  Cache slots past
    a sequence's length, and the spare block that unused block-table entries
    point at, are filled with ``pad_value`` so that any read of them shows up.
    """
    d = cfg.head_dim
    H, Hq, G, F = cfg.n_kv_heads, cfg.n_q_heads, cfg.group, cfg.n_fc
    assert Hq % H == 0 and 1 <= F <= d // 2
    kids = _seeds(cfg, seed)
    device = torch.device(device)

    rng = np.random.default_rng(kids[0])
    fc_idx = np.stack([np.sort(rng.choice(d // 2, size=F, replace=False)) for _ in range(H)])
    fc_idx = fc_idx.astype(np.int32)
    rng = np.random.default_rng(kids[1])
    massive = np.stack([np.sort(rng.choice(d, size=N_MASSIVE, replace=False)) for _ in range(H)])
    massive = massive.astype(np.int32)

    lens = draw_lengths(cfg, seed) if seq_lens is None else np.asarray(seq_lens, dtype=np.int32)
    assert lens.shape == (cfg.batch,) and (lens >= 0).all()
    nblk = [(int(t) + BLOCK - 1) // BLOCK for t in lens]
    max_blocks = max(1, max(nblk) if nblk else 1)
    n_used = int(sum(nblk))
    n_blocks = n_used + 1                         # + one spare block
    spare = n_blocks - 1
    rng = np.random.default_rng(kids[6])
    perm = rng.permutation(n_used).astype(np.int32)
    block_table = np.full((cfg.batch, max_blocks), spare, dtype=np.int32)
    o = 0
    for b, n in enumerate(nblk):
        block_table[b, :n] = perm[o:o + n]
        o += n

    scale = torch.ones(H, d, dtype=torch.float32, device=device)
    for g in range(H):
        scale[g, torch.as_tensor(massive[g], dtype=torch.long, device=device)] = MASSIVE_SCALE

    def gen(kid):
        gseed = int(np.random.default_rng(kid).integers(0, 2**62))
        gobj = torch.Generator(device=device)
        gobj.manual_seed(gseed)
        return gobj

    gq, gk, gv = gen(kids[2]), gen(kids[3]), gen(kids[4])
    dt = cfg.torch_dtype
    q = torch.empty(cfg.batch, Hq, d, dtype=dt, device=device)
    k_pool = torch.full((n_blocks, H, BLOCK, d), pad_value, dtype=dt, device=device)
    v_pool = torch.full((n_blocks, H, BLOCK, d), pad_value, dtype=dt, device=device)
    qscale = scale.repeat_interleave(G, dim=0)               # [Hq][d]

    for b in range(cfg.batch):
        t = int(lens[b])
        pos_q = torch.tensor([t], dtype=torch.int64, device=device)
        qb = torch.randn(Hq, 1, d, generator=gq, device=device) * qscale[:, None, :]
        q[b] = apply_rope(qb, pos_q, cfg.theta)[:, 0, :].to(dt)
        # Keys and values in chunks of whole blocks to bound temporary memory.
        chunk_blocks = max(1, (1 << 22) // (H * BLOCK * d))
        for k0 in range(0, nblk[b], chunk_blocks):
            k1 = min(nblk[b], k0 + chunk_blocks)
            j0, j1 = k0 * BLOCK, min(t, k1 * BLOCK)
            n = j1 - j0
            pos = torch.arange(j0, j1, dtype=torch.int64, device=device)
            kb = torch.randn(H, n, d, generator=gk, device=device) * scale[:, None, :]
            vb = torch.randn(H, n, d, generator=gv, device=device) * scale[:, None, :]
            kb = apply_rope(kb, pos, cfg.theta).to(dt)
            vb = vb.to(dt)
            for kk in range(k0, k1):
                p = int(block_table[b, kk])
                a, e = kk * BLOCK - j0, min(n, (kk + 1) * BLOCK - j0)
                k_pool[p, :, : e - a, :] = kb[:, a:e, :]
                v_pool[p, :, : e - a, :] = vb[:, a:e, :]

    return Inputs(cfg=cfg, seed=seed, seq_lens=lens, fc_idx=fc_idx, massive=massive,
                  block_table=block_table, n_blocks=n_blocks, q=q, k_pool=k_pool,
                  v_pool=v_pool)


def drifting_queries(q: torch.Tensor, n_steps: int, rho: float = 0.9, seed: int = 0) -> list:
    """Queries of n_steps consecutive decode steps that change every step:
    q_0 = q, q_{n+1} = rho q_n + sqrt(1 - rho^2) z_n, where z_n is Gaussian noise
    with the per-channel standard deviation of q (over sequences and heads),
    drawn from a seeded generator on q's device; rounded to q's dtype.  rho
    sets how much consecutive selections overlap."""
    gen = torch.Generator(device=q.device).manual_seed(0x5EED + seed)
    sd = q.float().std(dim=(0, 1), keepdim=True)
    out = [q.clone()]
    cur = q.float()
    for _ in range(n_steps - 1):
        z = torch.randn(q.shape, generator=gen, device=q.device, dtype=torch.float32) * sd
        cur = rho * cur + math.sqrt(1.0 - rho * rho) * z
        out.append(cur.to(q.dtype))
    return out


def random_scores(n_units: int, max_t: int, kind: str, seed: int = 0) -> np.ndarray:
    """Seeded fp32 score rows [n_units][max_t] for exercising the top-B select alone.

    kind: "normal" (continuous), "ties" (values from a tiny set: heavy exact ties),
    "const" (every score equal), "signed_zero" (mix of +0.0/-0.0 and a few values),
    "wide" (magnitudes spanning many binades, both signs), "sorted_asc" / "sorted_desc".
    """
    kinds = ["normal", "ties", "const", "signed_zero", "wide", "sorted_asc", "sorted_desc"]
    if kind not in kinds:
        raise ValueError(kind)
    rng = np.random.default_rng([BASE_SEED, 99, seed, kinds.index(kind)])
    shape = (n_units, max_t)
    if kind == "normal":
        x = rng.standard_normal(shape) * 11.0
    elif kind == "ties":
        x = rng.integers(-3, 4, size=shape).astype(np.float64) * 0.5
    elif kind == "const":
        x = np.full(shape, 1.25)
    elif kind == "signed_zero":
        x = np.where(rng.random(shape) < 0.5, 0.0, -0.0)
        m = rng.random(shape) < 0.01
        x[m] = rng.standard_normal(int(m.sum()))
    elif kind == "wide":
        x = rng.standard_normal(shape) * np.exp2(rng.integers(-60, 60, size=shape))
    elif kind == "sorted_asc":
        x = np.sort(rng.standard_normal(shape), axis=1)
    else:  # sorted_desc
        x = -np.sort(rng.standard_normal(shape), axis=1)
    return x.astype(np.float32)


def unit_rows(inp: Inputs, b: int, g: int, pool: torch.Tensor) -> torch.Tensor:
    """The first t_b cached rows [t_b][d] of kv head g of sequence b (plain indexing)."""
    t = int(inp.seq_lens[b])
    n = (t + BLOCK - 1) // BLOCK
    if n == 0:
        return pool.new_empty((0, pool.shape[-1]))
    idx = torch.as_tensor(inp.block_table[b, :n].astype(np.int64), device=pool.device)
    rows = pool[idx, g]                               # [n][256][d]
    return rows.reshape(n * BLOCK, -1)[:t]
