"""Plant plausible mistakes in a copy of the oracle (CPU only) and check that
at least one pin catches each: the pins are strong enough to trust the oracle."""
import importlib.util
import os
import types

import pytest

import oracle_pins as P

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "fasa_oracle.py")

# (name, text in the oracle, replacement)
MUTANTS = [
    ("tip_drops_odd_term",
     "S += q_group[h, 2 * i] * K[:, 2 * i] + q_group[h, 2 * i + 1] * K[:, 2 * i + 1]",
     "S += q_group[h, 2 * i] * K[:, 2 * i]"),
    ("tip_wrong_sign",
     "S += q_group[h, 2 * i] * K[:, 2 * i] + q_group[h, 2 * i + 1] * K[:, 2 * i + 1]",
     "S += q_group[h, 2 * i] * K[:, 2 * i] - q_group[h, 2 * i + 1] * K[:, 2 * i + 1]"),
    ("tip_wrong_index",
     "S += q_group[h, 2 * i] * K[:, 2 * i] + q_group[h, 2 * i + 1] * K[:, 2 * i + 1]",
     "S += q_group[h, i] * K[:, i] + q_group[h, i + 1] * K[:, i + 1]"),
    ("tip_swapped_pair",
     "S += q_group[h, 2 * i] * K[:, 2 * i] + q_group[h, 2 * i + 1] * K[:, 2 * i + 1]",
     "S += q_group[h, 2 * i] * K[:, 2 * i + 1] + q_group[h, 2 * i + 1] * K[:, 2 * i]"),
    ("tip_first_head_only",
     "for h in range(q_group.shape[0]):",
     "for h in range(1):"),
    ("topb_smallest",
     "order = np.lexsort((idx, -S[idx]))",
     "order = np.lexsort((idx, S[idx]))"),
    ("topb_tie_higher_index",
     "order = np.lexsort((idx, -S[idx]))",
     "order = np.lexsort((-idx, -S[idx]))"),
    ("topb_abs",
     "order = np.lexsort((idx, -S[idx]))",
     "order = np.lexsort((idx, -np.abs(S[idx])))"),
    ("topb_off_by_one",
     "n = min(int(budget), len(idx))",
     "n = min(int(budget) - 1, len(idx))"),
    ("forced_recent_off_by_one",
     "set(range(max(0, t - n_recent), t))",
     "set(range(max(0, t - n_recent + 1), t))"),
    ("forced_ignored",
     "    chosen, s_b = top_b(S, budget, forced)\n    sel = np.union1d(forced, chosen)",
     "    chosen, s_b = top_b(S, budget)\n    sel = np.union1d(forced, chosen)"),
    ("fac_no_scale",
     "z = (q_group @ K_sel.T) * scale",
     "z = (q_group @ K_sel.T)"),
    ("fac_default_scale_1_over_d",
     "scale = 1.0 / np.sqrt(d) if not scale else scale",
     "scale = 1.0 / d if not scale else scale"),
    ("fac_values_are_keys",
     "return p @ V_sel, p",
     "return p @ K_sel, p"),
    ("fac_softmax_wrong_axis",
     "p = e / e.sum(axis=1, keepdims=True)",
     "p = e / e.sum(axis=0, keepdims=True)"),
    ("rows_wrong_block",
     "out[j0:j0 + n] = pool[int(block_table_row[j0 // BLOCK]), g, :n, :]",
     "out[j0:j0 + n] = pool[int(block_table_row[0]), g, :n, :]"),
    ("dense_wrong_group_slice",
     "res[(b, g)] = fac(q[b, g * G:(g + 1) * G], K, V, scale)[0]",
     "res[(b, g)] = fac(q[b, g:g + G], K, V, scale)[0]"),
    ("dense_drops_last_token",
     "        res[(b, g)] = fac(q[b, g * G:(g + 1) * G], K, V, scale)[0]",
     "        res[(b, g)] = fac(q[b, g * G:(g + 1) * G], K[:-1], V[:-1], scale)[0]"),
    ("nondominant_keeps_odd_dominant",
     "        dominant.add(2 * int(i) + 1)\n",
     "        pass\n"),
    ("nondominant_wrong_pair_index",
     "        dominant.add(2 * int(i))\n",
     "        dominant.add(int(i))\n"),
    ("ca_pair_wrong_column",
     "out[1 + i] = qs[2 * i] * K[:, 2 * i] + qs[2 * i + 1] * K[:, 2 * i + 1]",
     "out[1 + i] = qs[2 * i] * K[:, 2 * i] + qs[2 * i + 1] * K[:, 2 * i]"),
    ("ca_first_head_only",
     "qs = q_group.sum(axis=0)",
     "qs = q_group[0]"),
    ("ca_full_drops_first_fc",
     "out[0] = K @ qs",
     "out[0] = K[:, 2:] @ qs[2:]"),
    ("decode_wrong_group_slice",
     "res[(b, g)] = decode_unit(q[b, g * G:(g + 1) * G], K, V, fc_idx[g], budget,",
     "res[(b, g)] = decode_unit(q[b, g:g + G], K, V, fc_idx[g], budget,"),
    ("decode_wrong_fc_row",
     "res[(b, g)] = decode_unit(q[b, g * G:(g + 1) * G], K, V, fc_idx[g], budget,",
     "res[(b, g)] = decode_unit(q[b, g * G:(g + 1) * G], K, V, fc_idx[0], budget,"),
    ("ca_divides_by_set_size",
     "ca[i] = len(full & set(fc_set.tolist())) / float(k_top)",
     "ca[i] = len(full & set(fc_set.tolist())) / float(max(len(full), 1))"),
    ("dominant_lowest_ca",
     "chosen, _ = top_b(np.asarray(mean_ca, dtype=np.float64), n_tip)",
     "chosen, _ = top_b(-np.asarray(mean_ca, dtype=np.float64), n_tip)"),
    ("tip_padding_slot_counted",
     "            if i < 0:\n                continue\n            S += q_group",
     "            S += q_group"),
    ("slab_swapped_pair",
     "out[f, :, 0] = K[:, 2 * fc[f]]",
     "out[f, :, 0] = K[:, 2 * fc[f] + 1]"),
]


def _load_mutant(old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, old
    src = src.replace(old, new)
    mod = types.ModuleType("fasa_oracle_mutant")
    exec(compile(src, "fasa_oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_some_pin_catches(name, old, new):
    mod = _load_mutant(old, new)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(mod)
        except Exception:
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passes every pin"
