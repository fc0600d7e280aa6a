"""The oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle_pins as P
from oracle import fasa_oracle as O


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(O)


def test_costmodel_reproduces_pages():
    P.check_costmodel_against_pages()


def test_oracle_on_generated_unit_is_consistent():
    """On a generated workload the oracle's selection has the requested size and
    its s_B separates chosen from unchosen scores."""
    from query_aware_sparse_fasa_amd import synth
    cfg = synth.CONFIGS["c2"].replace(batch=2, t=None, t_range=(300, 900), budget=40,
                                      n_sink=4, n_recent=16)
    inp = synth.make_inputs(cfg, seed=3)
    r = O.decode(inp.q.double().numpy(), inp.k_pool.double().numpy(), inp.v_pool.double().numpy(),
                 inp.block_table, inp.seq_lens, inp.fc_idx, cfg.budget, cfg.n_sink, cfg.n_recent)
    for (b, g), u in r.items():
        t = int(inp.seq_lens[b])
        forced = O.forced_tokens(t, cfg.n_sink, cfg.n_recent)
        assert len(u["sel"]) == len(forced) + min(cfg.budget, t - len(forced))
        rest = np.setdiff1d(np.arange(t), forced)
        chosen = np.setdiff1d(u["sel"], forced)
        unchosen = np.setdiff1d(rest, chosen)
        assert u["S"][chosen].min() >= u["s_B"] >= u["S"][unchosen].max()
        assert np.isfinite(u["out"]).all()
