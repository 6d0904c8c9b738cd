"""Mistakes planted on purpose into copies of the oracle's functions (on the
CPU): each must make at least one pin of ``test_oracle_pins.py`` fail.  This
shows the pins are strong enough to catch a dropped term, a wrong sign, a
wrong index or a transposed operand in the oracle."""
import inspect
import textwrap

import pytest

from oracle import pbsa_oracle as po
from oracle import rollout as orl
import test_oracle_pins as pins

# (function, source fragment, planted replacement, pins expected to catch it)
MUTATIONS = [
    ("attn_bwd", "dS = P * (dO @ V.T - D)", "dS = P * (dO @ V.T)",
     ["test_bwd_matches_central_finite_differences"]),
    ("attn_bwd", "dq[b, h, rows.start:rows.stop] = scale * (dS @ K)",
     "dq[b, h, rows.start:rows.stop] = (dS @ K)",
     ["test_bwd_matches_central_finite_differences"]),
    ("attn_bwd", "dV = P.T @ dO", "dV = P.T @ dO * scale",
     ["test_bwd_matches_central_finite_differences", "test_bwd_invariants"]),
    ("attn_bwd", "dK = scale * (dS.T @ Q)", "dK = scale * (P.T @ Q)",
     ["test_bwd_invariants", "test_bwd_matches_torch_autograd_dense_masked_form"]),
    ("attn_fwd", "lse[b, h, rows.start:rows.stop] = (m + np.log(l))[:, 0]",
     "lse[b, h, rows.start:rows.stop] = (np.log(l))[:, 0]",
     ["test_fwd_dense_limit_equals_textbook_attention", "test_fwd_golden_hand_example"]),
    ("attn_fwd", "z = scale * (q[b, h, rows.start:rows.stop] @ K.T)",
     "z = (q[b, h, rows.start:rows.stop] @ K.T)",
     ["test_fwd_dense_limit_equals_textbook_attention"]),
    ("attended_segments", 'seg.append(("cur", 0, nq))', 'seg.append(("cur", 0, nq - 1))',
     ["test_fwd_single_block_is_plain_attention", ("test_fwd_matches_bruteforce_token_mask", dict(T=4, d=8))]),
    ("attended_segments", 'for p in range(n_pool)]', 'for p in range(max(0, n_pool - 1))]',
     ["test_fwd_dense_limit_equals_textbook_attention"]),
    ("block_mean", "return rows.sum(axis=0) / n", "return rows.sum(axis=0) / max(n, 4)",
     ["test_block_mean_closed_form", "test_pooled_queries_ragged_tail"]),
    ("pooled_slots", "out[idx] = block_mean(k_slots[idx][:n])",
     "out[idx] = k_slots[idx][:n].sum(axis=0) / k_slots.shape[-2]",
     ["test_pooled_slots_ragged_closed_form"]),
    ("pooled_slots", "out[idx] = block_mean(k_slots[idx][:n])", "out[idx] = block_mean(k_slots[idx])",
     ["test_pooled_slots_ragged_closed_form"]),
    ("coarse_logit", "return float(scale * np.dot(_f64(qbar), _f64(kbar)))",
     "return float(np.dot(_f64(qbar), _f64(kbar)))",
     ["test_topk_scale_sign_matters", "test_coarse_scores_with_T1_are_token_logits"]),
    ("rank_key_desc", "return (0, -score, block_id)", "return (0, -score, -block_id)",
     ["test_topk_constructed_order_and_tiebreak", "test_update_ties_and_nan"]),
    ("rank_key_desc", "return (1, 0.0, block_id)", "return (-1, 0.0, block_id)",
     ["test_topk_constructed_order_and_tiebreak", "test_update_ties_and_nan"]),
    ("select", "pi = softmax(np.array(sp + [sw[w] for w in valid_w] + sc))",
     "pi = softmax(np.array(sp + [sw[w] for w in valid_w]))",
     ["test_mass_two_candidates_logistic", "test_mass_uniform_when_scores_equal"]),
    ("fine_mass", "P = e / e.sum(axis=1, keepdims=True)", "P = e",
     ["test_fine_mass_rows_sum_to_one", "test_fine_mass_uniform_when_queries_are_zero"]),
    ("fine_mass", "mass_win[b, h, slot] += m.sum()", "mass_win[b, h, min(slot + 1, W - 1)] += m.sum()",
     ["test_fine_mass_uniform_when_queries_are_zero", ("test_fine_mass_matches_bruteforce_token_mask", dict(T=4, d=8))]),
    ("fine_mass", "col_mass = P.sum(axis=0)", "col_mass = P.sum(axis=0) * 0 + P[0]",
     ["test_fine_mass_rows_sum_to_one"]),
    ("fine_mass", "z = scale * (q[b, h, rows.start:rows.stop] @ K.T)", "z = (q[b, h, rows.start:rows.stop] @ K.T)",
     [("test_fine_mass_matches_bruteforce_token_mask", dict(T=4, d=8))]),
    ("head_shared_masses", "tot[x] = tot.get(x, 0.0) + float(mass_pool[b, h, p])",
     "tot[x] = float(mass_pool[b, h, p])",
     ["test_update_head_shared_pool_is_best_subset_of_summed_mass"]),
    ("rollout.rollout_attention_grads", "dk[c][b, h, r] += dK[u]", "dk[t][b, h, r % Nq] += dK[u]",
     ["test_rollout_grads_match_autograd_of_flat_masked_attention"]),
    ("rollout.rollout_attention_grads", "dS = P * (dO @ V.T - Dr)", "dS = P * (dO @ V.T)",
     ["test_rollout_grads_match_autograd_of_flat_masked_attention",
      "test_rollout_grads_single_chunk_is_the_chunk_backward"]),
    ("rollout._history_rows", "r0, r1 = j * T, min(Nq, (j + 1) * T)", "r0, r1 = j * T, (j + 1) * T",
     ["test_rollout_grads_match_autograd_of_flat_masked_attention"]),
    ("memory_update_one", "free = sorted(free)", "free = sorted(free, reverse=True)",
     ["test_update_placement_golden"]),
    ("memory_update_one", "admitted = sorted([x for x in kept if x[0] == \"cand\"], key=lambda x: x[2])",
     "admitted = sorted([x for x in kept if x[0] == \"cand\"], key=lambda x: -x[2])",
     ["test_update_placement_golden"]),
    ("memory_update_one", "kept = pinned + rest[:C - len(pinned)]", "kept = pinned + rest[-(C - len(pinned)):]",
     ["test_update_matches_best_subset_bruteforce", "test_update_placement_golden"]),
]


def _module(fn_name):
    """'rollout.f' names a function of oracle/rollout.py, 'f' one of pbsa_oracle."""
    return (orl, fn_name.split(".", 1)[1]) if fn_name.startswith("rollout.") else (po, fn_name)


def _mutated(fn_name, old, new):
    mod, name = _module(fn_name)
    src = textwrap.dedent(inspect.getsource(getattr(mod, name)))
    assert old in src, (fn_name, old)
    ns = dict(vars(mod))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    return ns[name]


@pytest.mark.parametrize("fn_name,old,new,catchers", MUTATIONS,
                         ids=[f"{m[0]}:{i}" for i, m in enumerate(MUTATIONS)])
def test_pins_catch_planted_mistakes(monkeypatch, fn_name, old, new, catchers):
    mod, name = _module(fn_name)
    monkeypatch.setattr(mod, name, _mutated(fn_name, old, new))
    caught = []
    for name in catchers:
        name, kwargs = name if isinstance(name, tuple) else (name, {})
        try:
            getattr(pins, name)(**kwargs)
        except (AssertionError, ValueError, IndexError):
            caught.append(name)
    assert caught, f"no pin caught the mutation in {fn_name}: {new!r}"
