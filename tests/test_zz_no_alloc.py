"""fasa_decode_scratch (the allocation-free decode) against fasa_decode.  Needs a GPU.

Two calls in a row on the library's fixed scratch, the second with a smaller
input, each compared with fasa_decode on a workspace of its own: the same
selections bit for bit and the same outputs (the same kernels run).
"""
import sys

import numpy as np
import pytest
import torch

from query_aware_sparse_fasa_amd import fasa, synth
from query_aware_sparse_fasa_amd.workload import DeviceLayer

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _scratch_decode(L):
    out = torch.full_like(L.out, float("nan"))
    sel = torch.full_like(L.sel_idx, -7)
    cnt = torch.full_like(L.sel_count, -7)
    fasa.fasa_decode_scratch(L.shape, L.q, L.k_pool, L.v_pool, L.slab, L.block_table, L.seq_lens, L.max_t,
                             L.fc_idx, out, sel, cnt)
    return out, sel, cnt


@pytest.mark.parametrize("cases", [
    # (config, seed): an 8B-layer slice with ragged lengths (two-launch step),
    # then a smaller ragged batch with forced tokens.
    (("c2", dict(batch=3, t=None, t_range=(9000, 20000)), 3), ("c5", dict(batch=2, t_range=(700, 3000)), 5)),
    # Large budget (filter launch, separate select, split FAC), then the tiny fp32 workload.
    (("c3", dict(batch=2, t=None, t_range=(7000, 9000)), 7), ("c1", dict(), 1)),
    # The Qwen-shaped layer on the histogram-filtered lists (TIP's unit
    # histogram and arrival counters in the scratch), a 131072-token row, then
    # a shorter one.
    (("c4", dict(batch=1), 11), ("c4", dict(batch=1, t=None, t_range=(85000, 100000)), 13)),
])
def test_scratch_decode_matches_workspace_decode(cases):
    for k, (key, repl, seed) in enumerate(cases):
        cfg = synth.CONFIGS[key].replace(**repl)
        say(f"[scratch decode] call {k}: {cfg.name} batch {cfg.batch} seed {seed}")
        inp = synth.make_inputs(cfg, seed=seed)
        L = DeviceLayer(inp)
        assert fasa.fasa_workspace_size(L.shape, L.max_t) <= fasa.fasa_scratch_capacity()
        if key == "c4":
            assert fasa.fasa_decode_path(L.shape, L.max_t) == fasa.PATH_FILTERED_LISTS
        got = _scratch_decode(L)
        L.out.fill_(float("nan"))
        L.decode()
        torch.cuda.synchronize()
        assert torch.equal(got[2], L.sel_count), f"call {k}: sel_count differs"
        cap = L.cap
        assert torch.equal(got[1][..., :cap], L.sel_idx[..., :cap]), f"call {k}: sel_idx differs"
        assert torch.equal(got[0], L.out), f"call {k}: out differs (max {torch.nan_to_num(got[0] - L.out).abs().max()})"
        assert not torch.isnan(got[0]).any()
        del L, inp
