"""Device buffers for one decode layer, and calls of the C ABI on them.

Plumbing only: torch allocates device memory, the binding passes pointers.
Used by the tests, the benchmark and the smoke check.
"""
from __future__ import annotations

import numpy as np
import torch

from . import fasa
from .synth import Inputs


class DeviceLayer:
    """One decode layer's inputs and outputs resident on the GPU."""

    def __init__(self, inp: Inputs, device="cuda", with_slab: bool = True, build_slab: bool = True,
                 max_t: int = None):
        """max_t: the longest context the buffers are sized for (default: the inputs' longest)."""
        cfg = inp.cfg
        dev = torch.device(device)
        self.inp = inp
        self.cfg = cfg
        self.max_t = inp.max_t if max_t is None else max_t
        self.shape = fasa.make_shape(cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.n_fc, cfg.budget,
                                     inp.max_blocks, cfg.torch_dtype, cfg.n_sink, cfg.n_recent)
        fasa.fasa_check_fc_idx(self.shape, inp.fc_idx)
        self.q = inp.q.to(dev).contiguous()
        self.k_pool = inp.k_pool.to(dev).contiguous()
        self.v_pool = inp.v_pool.to(dev).contiguous()
        self.block_table = torch.from_numpy(inp.block_table).to(dev)
        self.seq_lens = torch.from_numpy(inp.seq_lens).to(dev)
        self.fc_idx = torch.from_numpy(inp.fc_idx).to(dev)
        self.cap = fasa.fasa_selection_capacity(self.shape, self.max_t)
        B, H, Hq = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads
        self.out = torch.zeros(B, Hq, 128, dtype=torch.float32, device=dev)
        self.sel_idx = torch.full((B, H, max(self.cap, 1)), -7, dtype=torch.int32, device=dev)
        self.sel_count = torch.full((B, H), -7, dtype=torch.int32, device=dev)
        self.scores = torch.full((B, H, max(self.max_t, 4)), float("nan"), dtype=torch.float32, device=dev)
        self.workspace = fasa.alloc_workspace(self.shape, self.max_t, device=dev)
        self.slab = None
        if with_slab:
            self.slab = fasa.alloc_slab(self.shape, device=dev)
            if build_slab:
                self.build_slab()

    # -- the C ABI on these buffers ---------------------------------------------------
    def build_slab(self, stream=None):
        fasa.fasa_slab_build(self.shape, self.k_pool, self.block_table, self.seq_lens, self.fc_idx,
                             self.slab, stream)

    def tip(self, use_slab=True, stream=None):
        fasa.fasa_tip(self.shape, self.q, self.slab if use_slab else None, self.k_pool, self.block_table,
                      self.seq_lens, self.fc_idx, self.scores, self.max_t, stream)

    def topk(self, scores=None, stream=None):
        fasa.fasa_topk(self.shape, self.scores if scores is None else scores, self.seq_lens, self.max_t,
                       self.sel_idx, self.sel_count, self.workspace, stream)

    def fac(self, stream=None):
        fasa.fasa_fac(self.shape, self.q, self.k_pool, self.v_pool, self.block_table, self.sel_idx,
                      self.sel_count, self.max_t, self.out, self.workspace, stream)

    def decode(self, use_slab=True, stream=None):
        fasa.fasa_decode(self.shape, self.q, self.k_pool, self.v_pool, self.slab if use_slab else None,
                         self.block_table, self.seq_lens, self.max_t, self.fc_idx, self.out,
                         self.sel_idx, self.sel_count, self.workspace, stream)

    def decode_tip(self, use_slab=True, stream=None):
        """fasa_decode's first launch only (TIP as the step runs it)."""
        fasa.fasa_decode_tip(self.shape, self.q, self.k_pool, self.slab if use_slab else None, self.block_table,
                             self.seq_lens, self.max_t, self.fc_idx, self.workspace, stream)

    def decode_rest(self, stream=None):
        fasa.fasa_decode_rest(self.shape, self.q, self.k_pool, self.v_pool, self.block_table, self.seq_lens,
                              self.max_t, self.out, self.sel_idx, self.sel_count, self.workspace, stream)

    def dense(self, out=None, stream=None):
        """Full attention over every cached token (into out, default self.dense_out)."""
        if getattr(self, "dense_ws", None) is None:
            self.dense_ws = fasa.alloc_dense_workspace(self.shape, self.max_t, device=self.q.device)
            self.dense_out = torch.zeros_like(self.out)
        fasa.fasa_dense_decode(self.shape, self.q, self.k_pool, self.v_pool, self.block_table, self.seq_lens,
                               self.max_t, self.dense_out if out is None else out, self.dense_ws, stream)

    def m_setup(self, stream=None):
        """FASA-M: pinned host arrays of this layer's non-dominant keys and values."""
        if getattr(self, "m_knd", None) is None:
            self.m_knd, self.m_v = fasa.alloc_m_host(self.shape, self.inp.n_blocks)
            n = fasa.fasa_m_workspace_size(self.shape, self.max_t)
            self.m_ws = torch.zeros(max(n, 256), dtype=torch.uint8, device=self.q.device)
            self.m_out = torch.zeros_like(self.out)
            self.m_sel_idx = torch.zeros_like(self.sel_idx)
            self.m_sel_count = torch.zeros_like(self.sel_count)
        fasa.fasa_m_offload(self.shape, self.k_pool, self.v_pool, self.block_table, self.seq_lens, self.fc_idx,
                            self.m_knd, self.m_v, stream)

    def m_decode(self, stream=None):
        fasa.fasa_m_decode(self.shape, self.q, self.slab, self.m_knd, self.m_v, self.block_table, self.seq_lens,
                           self.max_t, self.fc_idx, self.m_out, self.m_sel_idx, self.m_sel_count, self.m_ws, stream)

    def m_select(self, q=None, sel_idx=None, sel_count=None, stream=None):
        fasa.fasa_m_decode_select(self.shape, self.q if q is None else q, self.slab, self.block_table, self.seq_lens,
                                  self.max_t, self.fc_idx, self.m_sel_idx if sel_idx is None else sel_idx,
                                  self.m_sel_count if sel_count is None else sel_count, self.m_ws, stream)

    def m_prefetch(self, prev_sel_idx, prev_sel_count, parity, stream=None):
        fasa.fasa_m_prefetch(self.shape, self.slab, self.m_knd, self.m_v, self.block_table, self.max_t, self.fc_idx,
                             prev_sel_idx, prev_sel_count, parity, self.m_ws, stream)

    def m_finish(self, prev_sel_idx, prev_sel_count, parity, q=None, sel_idx=None, sel_count=None, hits=None,
                 stream=None):
        fasa.fasa_m_decode_finish(self.shape, self.q if q is None else q, self.slab, self.m_knd, self.m_v,
                                  self.block_table, self.max_t, self.fc_idx, prev_sel_idx, prev_sel_count,
                                  self.m_sel_idx if sel_idx is None else sel_idx,
                                  self.m_sel_count if sel_count is None else sel_count, parity, self.m_out,
                                  self.m_ws, hits, stream)

    # -- host copies ----------------------------------------------------------------
    def selection(self, b: int, g: int) -> np.ndarray:
        n = int(self.sel_count[b, g].item())
        return self.sel_idx[b, g, :n].cpu().numpy().astype(np.int64)

    def unit_host(self, b: int, g: int):
        """(q_group, K, V) of one unit as fp64 host arrays (from the generated inputs)."""
        from .synth import unit_rows
        G = self.cfg.group
        q = self.inp.q[b, g * G:(g + 1) * G].double().cpu().numpy()
        K = unit_rows(self.inp, b, g, self.inp.k_pool).double().cpu().numpy()
        V = unit_rows(self.inp, b, g, self.inp.v_pool).double().cpu().numpy()
        return q, K, V
