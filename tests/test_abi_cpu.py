"""The C ABI without a GPU: the library loads, exports what include/fasa.h
declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

from query_aware_sparse_fasa_amd import fasa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fasa.h")
FAKE = 0x10000   # never dereferenced: validation fails before any launch


def header_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\*|fasa_status|size_t)\s+(fasa_\w+)\s*\(", src, re.M)))


def test_exports_every_declared_symbol():
    L = fasa.lib()
    names = header_functions()
    assert len(names) == 28, names
    for n in names:
        assert hasattr(L, n), n
    assert sorted(fasa.EXPORTS) == names


def test_struct_layout_matches_header():
    assert ctypes.sizeof(fasa.fasa_shape) == 80
    assert fasa.fasa_shape.kv_block_stride.offset == 40
    assert fasa.fasa_shape.kv_dtype.offset == 72


def test_status_strings():
    for s in range(6):
        assert fasa.status_str(s).startswith("FASA_")
    assert "unknown" in fasa.status_str(99)


def good(**kw):
    base = dict(batch=2, n_q_heads=32, n_kv_heads=8, n_fc=16, budget=256, max_blocks_per_seq=16,
                kv_dtype=torch.bfloat16)
    base.update(kw)
    return fasa.make_shape(**base)


@pytest.mark.parametrize("key,max_t,path", [
    ("c1", 4096, fasa.PATH_LISTS), ("c2", 32768, fasa.PATH_LISTS), ("c3", 32768, fasa.PATH_SPLIT),
    ("c4", 131072, fasa.PATH_FILTERED_LISTS), ("c5", 65536, fasa.PATH_FILTER)])
def test_decode_path_of_each_workload(key, max_t, path):
    """The launch structure chosen for each workload at its full size (host
    logic only): lists at the single head and the 8B layer, filtered lists at
    the Qwen shape, the filter launch for the 512-unit ragged batch, the split
    FAC for the large budget."""
    from query_aware_sparse_fasa_amd import synth
    cfg = synth.CONFIGS[key]
    s = fasa.make_shape(cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.n_fc, cfg.budget, (max_t + 255) // 256,
                        cfg.torch_dtype, cfg.n_sink, cfg.n_recent)
    assert fasa.fasa_decode_path(s, max_t) == path
    assert fasa.fasa_decode_path(s, 0) == fasa.PATH_NONE


def test_decode_path_rejects_bad_arguments():
    s = good()
    assert fasa.lib().fasa_decode_path(ctypes.byref(s), 4096, None) == fasa.FASA_ERR_INVALID_ARG
    bad = good(n_fc=0)
    v = ctypes.c_int32()
    assert fasa.lib().fasa_decode_path(ctypes.byref(bad), 4096, ctypes.byref(v)) != 0
    assert fasa.lib().fasa_decode_path(ctypes.byref(s), 16 * 256 + 1, ctypes.byref(v)) != 0


def test_valid_shape_and_sizes():
    s = good()
    fasa.fasa_validate_shape(s)
    assert fasa.fasa_selection_capacity(s, 4096) == 256
    assert fasa.fasa_selection_capacity(s, 100) == 100
    s2 = good(n_sink=4, n_recent=64, budget=512)
    assert fasa.fasa_selection_capacity(s2, 4096) == 580
    assert fasa.fasa_selection_capacity(s, 0) == 0
    ws = fasa.fasa_workspace_size(s, 4096)
    assert ws >= 2 * 8 * 4096 * 4 and ws % 256 == 0


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 64, fasa.FASA_ERR_UNSUPPORTED),
    ("head_dim", 127, fasa.FASA_ERR_INVALID_ARG),
    ("block_size", 128, fasa.FASA_ERR_UNSUPPORTED),
    ("n_q_heads", 36, fasa.FASA_ERR_UNSUPPORTED),       # group 36/8 not integral -> invalid first
    ("n_fc", 0, fasa.FASA_ERR_INVALID_ARG),
    ("n_fc", 65, fasa.FASA_ERR_INVALID_ARG),
    ("budget", 0, fasa.FASA_ERR_INVALID_ARG),
    ("n_sink", -1, fasa.FASA_ERR_INVALID_ARG),
    ("n_recent", -5, fasa.FASA_ERR_INVALID_ARG),
    ("batch", 0, fasa.FASA_ERR_INVALID_ARG),
    ("batch", 70000, fasa.FASA_ERR_INVALID_ARG),
    ("n_kv_heads", 0, fasa.FASA_ERR_INVALID_ARG),
    ("kv_dtype", 7, fasa.FASA_ERR_INVALID_ARG),
    ("max_blocks_per_seq", 0, fasa.FASA_ERR_INVALID_ARG),
    ("kv_head_stride", 256 * 128 - 8, fasa.FASA_ERR_INVALID_ARG),
    ("kv_block_stride", 8 * 256 * 128 + 3, fasa.FASA_ERR_INVALID_ARG),
    ("slab_head_stride", 16 * 512 - 8, fasa.FASA_ERR_INVALID_ARG),
    ("slab_block_stride", 5, fasa.FASA_ERR_INVALID_ARG),
    ("scale", -1.0, fasa.FASA_ERR_INVALID_ARG),
    ("scale", float("nan"), fasa.FASA_ERR_INVALID_ARG),
])
def test_shape_rejections(field, value, status):
    s = good()
    setattr(s, field, value)
    if field == "n_q_heads":
        status = fasa.FASA_ERR_INVALID_ARG
    with pytest.raises(fasa.FasaError) as e:
        fasa.fasa_validate_shape(s)
    assert e.value.status == status


def test_group_limit():
    with pytest.raises(fasa.FasaError) as e:
        fasa.fasa_validate_shape(good(n_q_heads=64, n_kv_heads=2))
    assert e.value.status == fasa.FASA_ERR_UNSUPPORTED
    fasa.fasa_validate_shape(good(n_q_heads=32, n_kv_heads=2))


def test_fc_idx_check():
    s = good(n_kv_heads=2, n_q_heads=4, n_fc=3)
    fasa.fasa_check_fc_idx(s, [[0, 5, 63], [1, 2, 3]])
    fasa.fasa_check_fc_idx(s, [[0, 5, -1], [1, -1, -1]])      # per-head N_tip: trailing unused slots
    for bad in ([[0, 5, 64], [1, 2, 3]], [[0, 5, 5], [1, 2, 3]], [[0, 5, 6], [1, -1, 3]],
                [[-1, 5, 6], [1, 2, 3]], [[0, 5, -2], [1, 2, 3]], [[-1, -1, -1], [1, 2, 3]]):
        with pytest.raises(fasa.FasaError) as e:
            fasa.fasa_check_fc_idx(s, bad)
        assert e.value.status == fasa.FASA_ERR_INVALID_ARG


def raw(name, *args):
    return getattr(fasa.lib(), name)(*args)


def test_entry_points_reject_before_launch():
    s = good()
    sp = ctypes.byref(s)
    ws = fasa.fasa_workspace_size(s, 4096)
    E = fasa.FASA_ERR_INVALID_ARG
    # null pointers
    assert raw("fasa_tip", sp, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4096, None) == E
    assert raw("fasa_tip", sp, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, 4096, None) == E
    assert raw("fasa_topk", sp, None, FAKE, 4096, FAKE, FAKE, None, 0, None) == E
    assert raw("fasa_fac", sp, FAKE, FAKE, FAKE, FAKE, FAKE, None, 4096, FAKE, FAKE, ws, None) == E
    assert raw("fasa_slab_build", sp, FAKE, FAKE, FAKE, FAKE, None, None) == E
    assert raw("fasa_slab_append", sp, FAKE, FAKE, None, FAKE, FAKE, None) == E
    assert raw("fasa_decode", sp, FAKE, FAKE, FAKE, None, FAKE, FAKE, 4096, FAKE, None, FAKE, FAKE,
               FAKE, ws, None) == E
    # misaligned device pointers
    assert raw("fasa_tip", sp, FAKE, FAKE + 2, None, FAKE, FAKE, FAKE, FAKE, 4096, None) == E
    assert raw("fasa_tip", sp, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE + 4, 4096, None) == E
    # max_t out of range: negative, or more tokens than the block table can hold
    assert raw("fasa_tip", sp, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, -1, None) == E
    assert raw("fasa_tip", sp, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 16 * 256 + 1, None) == E
    # workspace missing, too small, misaligned
    W = fasa.FASA_ERR_WORKSPACE
    args = (sp, FAKE, FAKE, FAKE, None, FAKE, FAKE, 4096, FAKE, FAKE, FAKE, FAKE)
    assert raw("fasa_decode", *args, None, ws, None) == W
    assert raw("fasa_decode", *args, FAKE, ws - 1, None) == W
    assert raw("fasa_decode", *args, FAKE + 16, ws, None) == W
    assert raw("fasa_fac", sp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4096, FAKE, FAKE, 1024, None) == W
    # the two stages of the step: what each reads is checked, then the workspace
    tip_args = (sp, FAKE, FAKE, None, FAKE, FAKE, 4096)
    assert raw("fasa_decode_tip", *tip_args, None, FAKE, ws, None) == E          # fc_idx
    assert raw("fasa_decode_tip", sp, FAKE, None, None, FAKE, FAKE, 4096, FAKE, FAKE, ws, None) == E
    assert raw("fasa_decode_tip", sp, FAKE, FAKE, FAKE + 2, FAKE, FAKE, 4096, FAKE, FAKE, ws, None) == E
    assert raw("fasa_decode_tip", *tip_args, FAKE, FAKE, ws - 1, None) == W
    assert raw("fasa_decode_tip", *tip_args, FAKE, None, ws, None) == W
    rest = (sp, FAKE, FAKE, FAKE, FAKE, FAKE, 4096)
    assert raw("fasa_decode_rest", *rest, None, FAKE, FAKE, FAKE, ws, None) == E     # out
    assert raw("fasa_decode_rest", *rest, FAKE, None, FAKE, FAKE, ws, None) == E     # sel_idx, cap > 0
    assert raw("fasa_decode_rest", sp, FAKE, FAKE, None, FAKE, FAKE, 4096, FAKE, FAKE, FAKE, FAKE, ws,
               None) == E                                                            # v_pool
    assert raw("fasa_decode_rest", *rest, FAKE, FAKE, FAKE, FAKE + 16, ws, None) == W
    assert raw("fasa_decode_rest", sp, FAKE, FAKE, FAKE, FAKE, FAKE, -1, FAKE, FAKE, FAKE, FAKE, ws,
               None) == E                                                            # max_t
    # dense decode: null pointers, max_t, workspace
    dws = fasa.fasa_dense_workspace_size(s, 4096)
    assert raw("fasa_dense_decode", sp, FAKE, FAKE, FAKE, FAKE, None, 4096, FAKE, FAKE, dws, None) == E
    assert raw("fasa_dense_decode", sp, FAKE, FAKE, FAKE, FAKE, FAKE, 4096, None, FAKE, dws, None) == E
    assert raw("fasa_dense_decode", sp, FAKE + 2, FAKE, FAKE, FAKE, FAKE, 4096, FAKE, FAKE, dws, None) == E
    assert raw("fasa_dense_decode", sp, FAKE, FAKE, FAKE, FAKE, FAKE, -1, FAKE, FAKE, dws, None) == E
    assert raw("fasa_dense_decode", sp, FAKE, FAKE, FAKE, FAKE, FAKE, 4096, FAKE, FAKE, dws - 1, None) == W
    assert raw("fasa_dense_decode", sp, FAKE, FAKE, FAKE, FAKE, FAKE, 4096, FAKE, None, dws, None) == W
    assert raw("fasa_dense_decode", sp, FAKE, FAKE, FAKE, FAKE, FAKE, 4096, FAKE, FAKE + 16, dws, None) == W
    # sel_idx may be NULL only when the capacity is 0
    assert raw("fasa_topk", sp, FAKE, FAKE, 4096, None, FAKE, None, 0, None) == E
    # bad shape propagates
    s.head_dim = 64
    assert raw("fasa_decode", sp, FAKE, FAKE, FAKE, None, FAKE, FAKE, 4096, FAKE, FAKE, FAKE, FAKE,
               FAKE, ws, None) == fasa.FASA_ERR_UNSUPPORTED
    assert raw("fasa_workspace_size", sp, 4096, None) == fasa.FASA_ERR_UNSUPPORTED


def test_workspace_grows_with_context_and_batch():
    a = fasa.fasa_workspace_size(good(), 4096)
    b = fasa.fasa_workspace_size(good(max_blocks_per_seq=32), 8192)
    c = fasa.fasa_workspace_size(good(batch=4), 4096)
    assert b > a and c > a
    f32 = fasa.fasa_workspace_size(good(kv_dtype=torch.float32), 4096)
    assert f32 > a     # fp64 partials for fp32 caches
    d1 = fasa.fasa_dense_workspace_size(good(), 4096)
    d2 = fasa.fasa_dense_workspace_size(good(kv_dtype=torch.float32), 4096)
    assert d2 > d1 > 0  # fp64 partials for fp32 caches


def test_fasa_m_sizes_and_rejections():
    # host arrays: the non-dominant row is 128 - 2F elements padded to 16 bytes
    kb, vb = fasa.fasa_m_host_sizes(good(), 10)
    assert kb == 10 * 8 * 256 * 96 * 2 and vb == 10 * 8 * 256 * 128 * 2
    kb, _ = fasa.fasa_m_host_sizes(good(n_fc=5), 3)
    assert kb == 3 * 8 * 256 * 120 * 2            # 118 bf16 -> 120
    kb, _ = fasa.fasa_m_host_sizes(good(n_fc=5, kv_dtype=torch.float32), 3)
    assert kb == 3 * 8 * 256 * 120 * 4            # 118 fp32 -> 120
    kb, _ = fasa.fasa_m_host_sizes(good(n_fc=64), 1)
    assert kb == 0
    s = good()
    sp = ctypes.byref(s)
    assert fasa.fasa_m_workspace_size(s, 4096) > fasa.fasa_workspace_size(s, 4096)
    mws = fasa.fasa_m_workspace_size(s, 4096)
    E = fasa.FASA_ERR_INVALID_ARG
    n = ctypes.c_size_t()
    assert raw("fasa_m_host_sizes", sp, 0, ctypes.byref(n), ctypes.byref(n)) == E
    assert raw("fasa_m_offload", sp, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None) == E
    assert raw("fasa_m_offload", sp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 8, FAKE, None) == E
    args = [sp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4096, FAKE, FAKE, FAKE, FAKE, FAKE, mws, None]
    for k in (1, 2, 3, 4):                      # q, slab, k_nd, v missing
        bad = list(args)
        bad[k] = None
        assert raw("fasa_m_decode", *bad) == E
    bad = list(args)
    bad[7] = -1
    assert raw("fasa_m_decode", *bad) == E
    bad = list(args)
    bad[3] = FAKE + 4                           # misaligned host array
    assert raw("fasa_m_decode", *bad) == E
    # the stages of the prefetching step
    W = fasa.FASA_ERR_WORKSPACE
    sel = [sp, FAKE, FAKE, FAKE, FAKE, 4096, FAKE, FAKE, FAKE, FAKE, mws, None]
    assert raw("fasa_m_decode_select", *sel[:1], None, *sel[2:]) == E           # q
    assert raw("fasa_m_decode_select", *sel[:5], -1, *sel[6:]) == E              # max_t
    assert raw("fasa_m_decode_select", *sel[:10], mws - 1, None) == W
    pf = [sp, FAKE, FAKE, FAKE, FAKE, 4096, FAKE, FAKE, FAKE, 1, FAKE, mws, None]
    assert raw("fasa_m_prefetch", *pf[:2], None, *pf[3:]) == E                  # k_nd
    assert raw("fasa_m_prefetch", *pf[:8], None, *pf[9:]) == E                  # prev_sel_count
    assert raw("fasa_m_prefetch", *pf[:2], FAKE + 4, *pf[3:]) == E              # misaligned host array
    assert raw("fasa_m_prefetch", *pf[:9], 2, *pf[10:]) == E                    # parity
    fin = [sp, FAKE, FAKE, FAKE, FAKE, FAKE, 4096, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, mws, None]
    assert raw("fasa_m_decode_finish", *fin[:9], None, *fin[10:]) == E          # prev count without list
    assert raw("fasa_m_decode_finish", *fin[:8], None, None, *fin[10:]) == E    # hits without a previous list
    assert raw("fasa_m_decode_finish", *fin[:13], None, *fin[14:]) == E         # out
    assert raw("fasa_m_decode_finish", *fin[:6], -1, *fin[7:]) == E             # max_t
    assert raw("fasa_m_decode_finish", *fin[:12], -1, *fin[13:]) == E           # parity


def test_ca_sizes_and_rejections():
    s = good()
    sp = ctypes.byref(s)
    a = fasa.fasa_ca_workspace_size(s, 4096, 256)
    assert a > 0 and fasa.fasa_ca_workspace_size(s, 8192 // 2, 256) == a
    assert fasa.fasa_ca_workspace_size(good(max_blocks_per_seq=32), 8192, 256) > a
    E = fasa.FASA_ERR_INVALID_ARG
    n = ctypes.c_size_t()
    for k in (0, 4097):
        assert raw("fasa_ca_workspace_size", sp, 4096, k, ctypes.byref(n)) == E
        assert raw("fasa_ca_hits", sp, FAKE, FAKE, FAKE, FAKE, 4096, k, FAKE, None, FAKE, a, None) == E
    assert raw("fasa_ca_hits", sp, None, FAKE, FAKE, FAKE, 4096, 256, FAKE, None, FAKE, a, None) == E
    assert raw("fasa_ca_hits", sp, FAKE, FAKE, FAKE, FAKE, 4096, 256, None, None, FAKE, a, None) == E
    assert raw("fasa_ca_hits", sp, FAKE, FAKE, FAKE, FAKE, 4096, 256, FAKE, None, FAKE, a - 1, None) == \
        fasa.FASA_ERR_WORKSPACE
    for n_tip in (0, 65):
        assert raw("fasa_ca_dominant", sp, FAKE, 4, n_tip, FAKE, None) == E
    assert raw("fasa_ca_dominant", sp, FAKE, 0, 16, FAKE, None) == E
    assert raw("fasa_ca_dominant", sp, None, 4, 16, FAKE, None) == E


def test_binding_refuses_host_tensors():
    s = good()
    x = torch.zeros(4)
    with pytest.raises(ValueError):
        fasa.fasa_tip(s, x, x, None, x, x, x, x, 4)


def test_scratch_entry_rejects_calls_beyond_its_capacity():
    """fasa_decode_scratch: a workspace need above the fixed 64 MiB is refused on
    the host, before the device is touched; so is a bad shape."""
    assert fasa.fasa_scratch_capacity() == 64 << 20
    big = good(batch=64, max_blocks_per_seq=256)                 # 64 x 8 units x 65536 tokens
    assert fasa.fasa_workspace_size(big, 65536) > fasa.fasa_scratch_capacity()
    with pytest.raises(fasa.FasaError) as e:
        fasa.fasa_decode_scratch(big, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 65536, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert e.value.status == fasa.FASA_ERR_SCRATCH
    assert "64 MiB" in fasa.status_str(fasa.FASA_ERR_SCRATCH)
    with pytest.raises(fasa.FasaError) as e:
        fasa.fasa_decode_scratch(good(budget=0), FAKE, FAKE, FAKE,
                                 FAKE, FAKE, FAKE, 4096, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert e.value.status == fasa.FASA_ERR_INVALID_ARG
