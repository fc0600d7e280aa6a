"""Thin ctypes binding of libfasa.so (include/fasa.h).

Argument marshalling only: every function here checks tensor placement and
dtype, passes raw device pointers and the current HIP stream to the C entry
point of the same name, and raises ``FasaError`` on a non-OK status.  All
computation happens in the library's HIP kernels; if the library is missing
the first call raises -- there is no fallback.  PyTorch provides device memory
and streams only.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfasa.so")

FASA_OK, FASA_ERR_INVALID_ARG, FASA_ERR_UNSUPPORTED, FASA_ERR_WORKSPACE, FASA_ERR_HIP, FASA_ERR_SCRATCH = range(6)
FASA_F32, FASA_BF16 = 0, 1
HEAD_DIM = 128
BLOCK = 256

EXPORTS = ["fasa_status_str", "fasa_validate_shape", "fasa_selection_capacity",
           "fasa_workspace_size", "fasa_check_fc_idx", "fasa_slab_build", "fasa_slab_append",
           "fasa_tip", "fasa_topk", "fasa_fac", "fasa_decode", "fasa_decode_tip", "fasa_decode_rest",
           "fasa_decode_path",
           "fasa_dense_workspace_size",
           "fasa_dense_decode", "fasa_m_host_sizes", "fasa_m_offload", "fasa_m_workspace_size",
           "fasa_m_decode", "fasa_m_decode_select", "fasa_m_prefetch", "fasa_m_decode_finish",
           "fasa_ca_workspace_size", "fasa_ca_hits", "fasa_ca_dominant",
           "fasa_scratch_capacity", "fasa_decode_scratch"]


class fasa_shape(ctypes.Structure):
    """Mirror of the C struct fasa_shape."""

    _fields_ = [
        ("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("n_fc", ctypes.c_int32), ("budget", ctypes.c_int32),
        ("n_sink", ctypes.c_int32), ("n_recent", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32), ("kv_block_stride", ctypes.c_int64),
        ("kv_head_stride", ctypes.c_int64), ("slab_block_stride", ctypes.c_int64),
        ("slab_head_stride", ctypes.c_int64), ("kv_dtype", ctypes.c_int32), ("scale", ctypes.c_float),
    ]


class FasaError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__(f"{fn}: {status_str(status)}")


_lib = None
_P = ctypes.c_void_p
_S = ctypes.POINTER(fasa_shape)
_I32 = ctypes.c_int32


def lib() -> ctypes.CDLL:
    """Load libfasa.so (once).  Importing torch first makes the library bind to
    torch's HIP runtime, so both share one device context and its streams."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise FileNotFoundError(
            f"{LIB_PATH} is missing: build it with `python -m query_aware_sparse_fasa_amd.build` "
            "(there is no CPU fallback)")
    L = ctypes.CDLL(LIB_PATH)
    sig = {
        "fasa_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "fasa_validate_shape": (ctypes.c_int, [_S]),
        "fasa_selection_capacity": (ctypes.c_int, [_S, _I32, ctypes.POINTER(_I32)]),
        "fasa_workspace_size": (ctypes.c_int, [_S, _I32, ctypes.POINTER(ctypes.c_size_t)]),
        "fasa_check_fc_idx": (ctypes.c_int, [_S, _P]),
        "fasa_slab_build": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P]),
        "fasa_slab_append": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P]),
        "fasa_tip": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _P, _I32, _P]),
        "fasa_topk": (ctypes.c_int, [_S, _P, _P, _I32, _P, _P, _P, ctypes.c_size_t, _P]),
        "fasa_fac": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _I32, _P, _P, ctypes.c_size_t, _P]),
        "fasa_decode": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _P, _P,
                                       ctypes.c_size_t, _P]),
        "fasa_decode_tip": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _I32, _P, _P, ctypes.c_size_t, _P]),
        "fasa_decode_rest": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _P, ctypes.c_size_t,
                                            _P]),
        "fasa_decode_path": (ctypes.c_int, [_S, _I32, ctypes.POINTER(ctypes.c_int32)]),
        "fasa_dense_workspace_size": (ctypes.c_int, [_S, _I32, ctypes.POINTER(ctypes.c_size_t)]),
        "fasa_dense_decode": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _I32, _P, _P, ctypes.c_size_t, _P]),
        "fasa_m_host_sizes": (ctypes.c_int, [_S, ctypes.c_int64, ctypes.POINTER(ctypes.c_size_t),
                                             ctypes.POINTER(ctypes.c_size_t)]),
        "fasa_m_offload": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _P, _P]),
        "fasa_m_workspace_size": (ctypes.c_int, [_S, _I32, ctypes.POINTER(ctypes.c_size_t)]),
        "fasa_m_decode": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _P, _P,
                                         ctypes.c_size_t, _P]),
        "fasa_ca_workspace_size": (ctypes.c_int, [_S, _I32, _I32, ctypes.POINTER(ctypes.c_size_t)]),
        "fasa_m_decode_select": (ctypes.c_int, [_S, _P, _P, _P, _P, _I32, _P, _P, _P, _P, ctypes.c_size_t, _P]),
        "fasa_m_prefetch": (ctypes.c_int, [_S, _P, _P, _P, _P, _I32, _P, _P, _P, _I32, _P, ctypes.c_size_t, _P]),
        "fasa_m_decode_finish": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _P, _P, _I32, _P, _P, _P,
                                                ctypes.c_size_t, _P]),
        "fasa_ca_hits": (ctypes.c_int, [_S, _P, _P, _P, _P, _I32, _I32, _P, _P, _P, ctypes.c_size_t, _P]),
        "fasa_ca_dominant": (ctypes.c_int, [_S, _P, _I32, _I32, _P, _P]),
        "fasa_scratch_capacity": (ctypes.c_size_t, []),
        "fasa_decode_scratch": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _P, _P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def status_str(status: int) -> str:
    return lib().fasa_status_str(int(status)).decode()


def _check(status: int, fn: str):
    if status != FASA_OK:
        raise FasaError(status, fn)


# --------------------------------------------------------------------------- shapes
def make_shape(batch: int, n_q_heads: int, n_kv_heads: int, n_fc: int, budget: int,
               max_blocks_per_seq: int, kv_dtype: torch.dtype, n_sink: int = 0, n_recent: int = 0,
               scale: float = 0.0, kv_block_stride: Optional[int] = None,
               kv_head_stride: Optional[int] = None, slab_block_stride: Optional[int] = None,
               slab_head_stride: Optional[int] = None) -> fasa_shape:
    """A shape for a paged pool [n_blocks][H_kv][256][128] and a slab
    [batch][max_blocks_per_seq][H_kv][F][256][2] unless other strides are given."""
    s = fasa_shape()
    s.batch, s.n_q_heads, s.n_kv_heads, s.head_dim = batch, n_q_heads, n_kv_heads, HEAD_DIM
    s.n_fc, s.budget, s.n_sink, s.n_recent = n_fc, budget, n_sink, n_recent
    s.block_size, s.max_blocks_per_seq = BLOCK, max_blocks_per_seq
    s.kv_head_stride = BLOCK * HEAD_DIM if kv_head_stride is None else kv_head_stride
    s.kv_block_stride = n_kv_heads * BLOCK * HEAD_DIM if kv_block_stride is None else kv_block_stride
    s.slab_head_stride = n_fc * 2 * BLOCK if slab_head_stride is None else slab_head_stride
    s.slab_block_stride = n_kv_heads * n_fc * 2 * BLOCK if slab_block_stride is None else slab_block_stride
    s.kv_dtype = {torch.float32: FASA_F32, torch.bfloat16: FASA_BF16}[kv_dtype]
    s.scale = scale
    return s


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"expected a torch.Tensor, got {type(x)}")
    if not x.is_cuda:
        raise ValueError("FASA buffers must be device (cuda/hip) tensors")
    if not x.is_contiguous():
        raise ValueError("FASA buffers must be contiguous")
    return x.data_ptr()


def _need(x, dtype, name):
    if isinstance(x, torch.Tensor) and x.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {x.dtype}")


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# --------------------------------------------------------------------------- entry points
def fasa_validate_shape(shape: fasa_shape) -> None:
    _check(lib().fasa_validate_shape(ctypes.byref(shape)), "fasa_validate_shape")


def fasa_selection_capacity(shape: fasa_shape, max_t: int) -> int:
    cap = _I32()
    _check(lib().fasa_selection_capacity(ctypes.byref(shape), max_t, ctypes.byref(cap)),
           "fasa_selection_capacity")
    return cap.value


def fasa_workspace_size(shape: fasa_shape, max_t: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().fasa_workspace_size(ctypes.byref(shape), max_t, ctypes.byref(n)), "fasa_workspace_size")
    return n.value


# Launch structures reported by fasa_decode_path (the header's FASA_PATH_* values).
PATH_NONE, PATH_LISTS, PATH_FILTERED_LISTS, PATH_FILTER, PATH_SPLIT = 0, 1, 2, 3, 4


def fasa_decode_path(shape: fasa_shape, max_t: int) -> int:
    v = ctypes.c_int32()
    _check(lib().fasa_decode_path(ctypes.byref(shape), max_t, ctypes.byref(v)), "fasa_decode_path")
    return v.value


def fasa_check_fc_idx(shape: fasa_shape, fc_idx_host) -> None:
    a = np.ascontiguousarray(np.asarray(fc_idx_host, dtype=np.int32))
    _check(lib().fasa_check_fc_idx(ctypes.byref(shape), a.ctypes.data), "fasa_check_fc_idx")


def fasa_slab_build(shape, k_pool, block_table, seq_lens, fc_idx, slab, stream=None) -> None:
    for x, n in ((block_table, "block_table"), (seq_lens, "seq_lens"), (fc_idx, "fc_idx")):
        _need(x, torch.int32, n)
    _check(lib().fasa_slab_build(ctypes.byref(shape), _ptr(k_pool), _ptr(block_table), _ptr(seq_lens),
                                 _ptr(fc_idx), _ptr(slab), _stream(stream)), "fasa_slab_build")


def fasa_slab_append(shape, k_pool, block_table, positions, fc_idx, slab, stream=None) -> None:
    for x, n in ((block_table, "block_table"), (positions, "positions"), (fc_idx, "fc_idx")):
        _need(x, torch.int32, n)
    _check(lib().fasa_slab_append(ctypes.byref(shape), _ptr(k_pool), _ptr(block_table), _ptr(positions),
                                  _ptr(fc_idx), _ptr(slab), _stream(stream)), "fasa_slab_append")


def fasa_tip(shape, q, slab, k_pool, block_table, seq_lens, fc_idx, scores, max_t, stream=None) -> None:
    _need(scores, torch.float32, "scores")
    _check(lib().fasa_tip(ctypes.byref(shape), _ptr(q), _ptr(slab), _ptr(k_pool), _ptr(block_table),
                          _ptr(seq_lens), _ptr(fc_idx), _ptr(scores), max_t, _stream(stream)), "fasa_tip")


def fasa_topk(shape, scores, seq_lens, max_t, sel_idx, sel_count, workspace=None, stream=None) -> None:
    _need(scores, torch.float32, "scores")
    _need(sel_idx, torch.int32, "sel_idx")
    _need(sel_count, torch.int32, "sel_count")
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fasa_topk(ctypes.byref(shape), _ptr(scores), _ptr(seq_lens), max_t, _ptr(sel_idx),
                           _ptr(sel_count), _ptr(workspace), nbytes, _stream(stream)), "fasa_topk")


def fasa_fac(shape, q, k_pool, v_pool, block_table, sel_idx, sel_count, max_t, out, workspace,
             stream=None) -> None:
    _need(out, torch.float32, "out")
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().fasa_fac(ctypes.byref(shape), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                          _ptr(sel_idx), _ptr(sel_count), max_t, _ptr(out), _ptr(workspace), nbytes,
                          _stream(stream)), "fasa_fac")


def fasa_decode(shape, q, k_pool, v_pool, slab, block_table, seq_lens, max_t, fc_idx, out, sel_idx,
                sel_count, workspace, stream=None) -> None:
    _need(out, torch.float32, "out")
    _need(sel_idx, torch.int32, "sel_idx")
    _need(sel_count, torch.int32, "sel_count")
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().fasa_decode(ctypes.byref(shape), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(slab),
                             _ptr(block_table), _ptr(seq_lens), max_t, _ptr(fc_idx), _ptr(out),
                             _ptr(sel_idx), _ptr(sel_count), _ptr(workspace), nbytes, _stream(stream)),
           "fasa_decode")


def fasa_decode_tip(shape, q, k_pool, slab, block_table, seq_lens, max_t, fc_idx, workspace, stream=None) -> None:
    """The first launch of fasa_decode (TIP with what the rest of the step reads)."""
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().fasa_decode_tip(ctypes.byref(shape), _ptr(q), _ptr(k_pool), _ptr(slab), _ptr(block_table),
                                 _ptr(seq_lens), max_t, _ptr(fc_idx), _ptr(workspace), nbytes, _stream(stream)),
           "fasa_decode_tip")


def fasa_decode_rest(shape, q, k_pool, v_pool, block_table, seq_lens, max_t, out, sel_idx, sel_count, workspace,
                     stream=None) -> None:
    """The rest of fasa_decode after fasa_decode_tip (top-B and FAC)."""
    _need(out, torch.float32, "out")
    _need(sel_idx, torch.int32, "sel_idx")
    _need(sel_count, torch.int32, "sel_count")
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().fasa_decode_rest(ctypes.byref(shape), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                                  _ptr(seq_lens), max_t, _ptr(out), _ptr(sel_idx), _ptr(sel_count),
                                  _ptr(workspace), nbytes, _stream(stream)), "fasa_decode_rest")


def fasa_scratch_capacity() -> int:
    return int(lib().fasa_scratch_capacity())


def fasa_decode_scratch(shape, q, k_pool, v_pool, slab, block_table, seq_lens, max_t, fc_idx, out, sel_idx,
                        sel_count, stream=None) -> None:
    """fasa_decode with the library's own fixed device scratch as workspace."""
    _need(out, torch.float32, "out")
    _need(sel_idx, torch.int32, "sel_idx")
    _need(sel_count, torch.int32, "sel_count")
    _check(lib().fasa_decode_scratch(ctypes.byref(shape), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(slab),
                                     _ptr(block_table), _ptr(seq_lens), max_t, _ptr(fc_idx), _ptr(out),
                                     _ptr(sel_idx), _ptr(sel_count), _stream(stream)), "fasa_decode_scratch")


def fasa_dense_workspace_size(shape: fasa_shape, max_t: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().fasa_dense_workspace_size(ctypes.byref(shape), max_t, ctypes.byref(n)),
           "fasa_dense_workspace_size")
    return n.value


def fasa_dense_decode(shape, q, k_pool, v_pool, block_table, seq_lens, max_t, out, workspace,
                      stream=None) -> None:
    _need(out, torch.float32, "out")
    _need(block_table, torch.int32, "block_table")
    _need(seq_lens, torch.int32, "seq_lens")
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().fasa_dense_decode(ctypes.byref(shape), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                   _ptr(block_table), _ptr(seq_lens), max_t, _ptr(out), _ptr(workspace),
                                   nbytes, _stream(stream)), "fasa_dense_decode")


def _host_ptr(x) -> Optional[int]:
    """Pointer of a pinned host tensor (FASA-M's host arrays)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"expected a torch.Tensor, got {type(x)}")
    if x.is_cuda or not x.is_pinned():
        raise ValueError("FASA-M host arrays must be pinned host tensors (pin_memory=True)")
    if not x.is_contiguous():
        raise ValueError("FASA buffers must be contiguous")
    return x.data_ptr()


def fasa_m_host_sizes(shape: fasa_shape, n_blocks: int):
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().fasa_m_host_sizes(ctypes.byref(shape), n_blocks, ctypes.byref(a), ctypes.byref(b)),
           "fasa_m_host_sizes")
    return a.value, b.value


def fasa_m_offload(shape, k_pool, v_pool, block_table, seq_lens, fc_idx, k_nd_host, v_host, stream=None) -> None:
    for x, n in ((block_table, "block_table"), (seq_lens, "seq_lens"), (fc_idx, "fc_idx")):
        _need(x, torch.int32, n)
    _check(lib().fasa_m_offload(ctypes.byref(shape), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                                _ptr(seq_lens), _ptr(fc_idx), _host_ptr(k_nd_host), _host_ptr(v_host),
                                _stream(stream)), "fasa_m_offload")


def fasa_m_workspace_size(shape: fasa_shape, max_t: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().fasa_m_workspace_size(ctypes.byref(shape), max_t, ctypes.byref(n)), "fasa_m_workspace_size")
    return n.value


def fasa_m_decode(shape, q, slab, k_nd_host, v_host, block_table, seq_lens, max_t, fc_idx, out, sel_idx,
                  sel_count, workspace, stream=None) -> None:
    _need(out, torch.float32, "out")
    _need(sel_idx, torch.int32, "sel_idx")
    _need(sel_count, torch.int32, "sel_count")
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().fasa_m_decode(ctypes.byref(shape), _ptr(q), _ptr(slab), _host_ptr(k_nd_host), _host_ptr(v_host),
                               _ptr(block_table), _ptr(seq_lens), max_t, _ptr(fc_idx), _ptr(out), _ptr(sel_idx),
                               _ptr(sel_count), _ptr(workspace), nbytes, _stream(stream)), "fasa_m_decode")


def fasa_m_decode_select(shape, q, slab, block_table, seq_lens, max_t, fc_idx, sel_idx, sel_count, workspace,
                         stream=None) -> None:
    """FASA-M stage 1: TIP on the slab and the exact top-B."""
    _need(sel_idx, torch.int32, "sel_idx")
    _need(sel_count, torch.int32, "sel_count")
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().fasa_m_decode_select(ctypes.byref(shape), _ptr(q), _ptr(slab), _ptr(block_table), _ptr(seq_lens),
                                      max_t, _ptr(fc_idx), _ptr(sel_idx), _ptr(sel_count), _ptr(workspace), nbytes,
                                      _stream(stream)), "fasa_m_decode_select")


def fasa_m_prefetch(shape, slab, k_nd_host, v_host, block_table, max_t, fc_idx, prev_sel_idx, prev_sel_count,
                    parity, workspace, stream=None) -> None:
    """The rows of a previous selection into row area 1 - parity, for a step of that parity."""
    _need(prev_sel_idx, torch.int32, "prev_sel_idx")
    _need(prev_sel_count, torch.int32, "prev_sel_count")
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().fasa_m_prefetch(ctypes.byref(shape), _ptr(slab), _host_ptr(k_nd_host), _host_ptr(v_host),
                                 _ptr(block_table), max_t, _ptr(fc_idx), _ptr(prev_sel_idx), _ptr(prev_sel_count),
                                 parity, _ptr(workspace), nbytes, _stream(stream)), "fasa_m_prefetch")


def fasa_m_decode_finish(shape, q, slab, k_nd_host, v_host, block_table, max_t, fc_idx, prev_sel_idx,
                         prev_sel_count, sel_idx, sel_count, parity, out, workspace, hits=None, stream=None) -> None:
    """FASA-M stage 2: rows into row area `parity` (the previous selection's from the other area), then FAC."""
    _need(out, torch.float32, "out")
    _need(sel_idx, torch.int32, "sel_idx")
    _need(sel_count, torch.int32, "sel_count")
    _need(prev_sel_idx, torch.int32, "prev_sel_idx")
    _need(prev_sel_count, torch.int32, "prev_sel_count")
    _need(hits, torch.int32, "hits")
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().fasa_m_decode_finish(ctypes.byref(shape), _ptr(q), _ptr(slab), _host_ptr(k_nd_host),
                                      _host_ptr(v_host), _ptr(block_table), max_t, _ptr(fc_idx), _ptr(prev_sel_idx),
                                      _ptr(prev_sel_count), _ptr(sel_idx), _ptr(sel_count), parity, _ptr(out),
                                      _ptr(hits), _ptr(workspace), nbytes, _stream(stream)), "fasa_m_decode_finish")


def fasa_ca_workspace_size(shape: fasa_shape, max_t: int, k_top: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().fasa_ca_workspace_size(ctypes.byref(shape), max_t, k_top, ctypes.byref(n)),
           "fasa_ca_workspace_size")
    return n.value


def fasa_ca_hits(shape, q, k_pool, block_table, seq_lens, max_t, k_top, hits, workspace, stream=None,
                 topk=None) -> None:
    """topk (optional, int32 [batch][H_kv][65][min(k_top, max_t)]): the top-K lists behind the counts."""
    _need(hits, torch.int32, "hits")
    _need(block_table, torch.int32, "block_table")
    _need(seq_lens, torch.int32, "seq_lens")
    _need(topk, torch.int32, "topk")
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().fasa_ca_hits(ctypes.byref(shape), _ptr(q), _ptr(k_pool), _ptr(block_table), _ptr(seq_lens), max_t,
                              k_top, _ptr(hits), _ptr(topk), _ptr(workspace), nbytes, _stream(stream)),
           "fasa_ca_hits")


def fasa_ca_dominant(shape, hits, n_rows, n_tip, fc_idx, stream=None) -> None:
    _need(hits, torch.int32, "hits")
    _need(fc_idx, torch.int32, "fc_idx")
    _check(lib().fasa_ca_dominant(ctypes.byref(shape), _ptr(hits), n_rows, n_tip, _ptr(fc_idx), _stream(stream)),
           "fasa_ca_dominant")


# --------------------------------------------------------------------------- buffers
def alloc_slab(shape: fasa_shape, device="cuda") -> torch.Tensor:
    """The dominant-key cache, indexed by (sequence, logical block):
    [batch][max_blocks_per_seq][H_kv][F][256][2] in the cache dtype."""
    dt = torch.bfloat16 if shape.kv_dtype == FASA_BF16 else torch.float32
    return torch.empty(shape.batch, shape.max_blocks_per_seq, shape.n_kv_heads, shape.n_fc, BLOCK, 2, dtype=dt,
                       device=device)


def alloc_m_host(shape: fasa_shape, n_blocks: int):
    """Pinned host arrays (k_nd, v) of FASA-M for a pool of n_blocks blocks."""
    kb, vb = fasa_m_host_sizes(shape, n_blocks)
    dt = torch.bfloat16 if shape.kv_dtype == FASA_BF16 else torch.float32
    es = 2 if shape.kv_dtype == FASA_BF16 else 4
    nd = kb // es // (n_blocks * shape.n_kv_heads * BLOCK)
    k_nd = torch.zeros(n_blocks, shape.n_kv_heads, BLOCK, nd, dtype=dt, pin_memory=True)
    v = torch.zeros(n_blocks, shape.n_kv_heads, BLOCK, HEAD_DIM, dtype=dt, pin_memory=True)
    assert k_nd.numel() * es == kb and v.numel() * es == vb
    return k_nd, v


def alloc_dense_workspace(shape: fasa_shape, max_t: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(fasa_dense_workspace_size(shape, max_t), 256), dtype=torch.uint8, device=device)


def alloc_workspace(shape: fasa_shape, max_t: int, device="cuda") -> torch.Tensor:
    """Zero-filled, so the select takes its fast path from the first call."""
    n = fasa_workspace_size(shape, max_t)
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)
