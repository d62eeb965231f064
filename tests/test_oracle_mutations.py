"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
in ``test_oracle_pins.py`` catch every one of them.

Each mutation is a one-place edit of the oracle's source (a dropped term, a
wrong sign or index, a transposed operand, a wrong reduction). The mutated
source is loaded as a fresh module and the pins run against it; at least one
pin must fail. This checks the pins themselves, not the HIP path.
"""
import inspect
import os
import types

import pytest

import oracle.msa_oracle as O
import tests.test_oracle_pins as P

SRC = open(inspect.getsourcefile(O)).read()

MUTATIONS = {
    "bf16_truncates": ("np.rint(np.ldexp(m[normal], 8))", "np.trunc(np.ldexp(m[normal], 8))"),
    "plan_floor": ("(int(L) + chunk - 1) // chunk", "int(L) // chunk + 1"),
    "rope_sign": ("lo * c - hi * s, hi * c + lo * s", "lo * c + hi * s, hi * c - lo * s"),
    "rope_adjacent_pairs": ("lo, hi = x[..., :half], x[..., half:]", "lo, hi = x[..., 0::2], x[..., 1::2]"),
    "rope_frequency": ("omega = theta ** (-2.0 * np.arange(half, dtype=np.float64) / Dh)",
                       "omega = theta ** (-1.0 * np.arange(half, dtype=np.float64) / Dh)"),
    "pool_divides_by_P": ("kbar = k[a:b].sum(axis=0) / (b - a)", "kbar = k[a:b].sum(axis=0) / chunk"),
    "pool_v_divides_by_P": ("f64_to_bf16(v[a:b].sum(axis=0) / (b - a))", "f64_to_bf16(v[a:b].sum(axis=0) / chunk)"),
    "pool_global_positions": ("local_pos = np.arange(t1 - t0)", "local_pos = np.arange(t0, t1)"),
    "pool_rotates_router_keys": ("kr = bf16_to_f64(KR[t0:t1])",
                                 "kr = rope_rotate(bf16_to_f64(KR[t0:t1]), np.arange(t1 - t0), theta)"),
    "pool_chunk_mode_position": ("kbar = rope_rotate(kbar[None], np.array([c]), theta)[0]",
                                 "kbar = rope_rotate(kbar[None], np.array([c * chunk]), theta)[0]"),
    "route_sums_heads": ("return cos.sum(axis=-1) / H", "return cos.sum(axis=-1)"),
    "route_unnormalised_keys": ("k = _unit(bf16_to_f64(KRbar))", "k = bf16_to_f64(KRbar)"),
    "route_mean_over_tokens": ("if token_reduce == TOKEN_REDUCE_MAX:", "if token_reduce != TOKEN_REDUCE_MAX:"),
    "route_transposed_heads": ('cos = np.einsum("mhd,chd->mch", q, k)', 'cos = np.einsum("mhd,chd->mch", q, k[:, ::-1])'),
    "doc_mean_of_chunks": ("S_c[dco[i]:dco[i + 1]].max()", "S_c[dco[i]:dco[i + 1]].mean()"),
    "topk_ties_to_highest_id": ("else 0.0, i))", "else 0.0, -i))"),
    "merge_replaces": ("s = np.maximum(np.asarray(prev_doc_scores, dtype=np.float64), s)", "s = s"),
    "attend_no_causal_mask": ("n_vis = q_local_idx[u] + 1", "n_vis = M_loc"),
    "attend_pos0_zero": ("pos0 = len(sel_ids)", "pos0 = 0"),
    "attend_gqa_modulo": ("g = h // group", "g = h % Hkv"),
    "attend_scale_1_over_D": ("scale = 1.0 / math.sqrt(Dh)", "scale = 1.0 / Dh"),
    "attend_query_positions": ("q_local_idx = np.arange(M_loc - M, M_loc)", "q_local_idx = np.arange(0, M)"),
    "attend_rotates_pre_rotated": ("    if not k_loc_rotated:\n        kl = rope_rotate",
                                   "    if True:\n        kl = rope_rotate"),
    "attend_values_from_keys": ("vals = np.concatenate([vmem[:, g, :], vl[:n_vis, g, :]], axis=0)",
                                "vals = np.concatenate([kmem[:, g, :], vl[:n_vis, g, :]], axis=0)"),
    "aux_no_projection": ("kh[c] - ch[:, None] * qh[t], kh[c])", "kh[c], kh[c])"),
    "aux_key_grad_swapped": ("qh[t] - ch[:, None] * kh[c], qh[t])", "kh[c] - ch[:, None] * qh[t], qh[t])"),
    "aux_negatives_include_positives": ("neg[P] = False", "neg[P] = True"),
    "aux_missing_temperature": ("ds[neg] += e[neg] / z / tau", "ds[neg] += e[neg] / z"),
    "aux_sum_not_mean": ("    loss /= len(P)\n    ds /= len(P)", "    pass"),
    "aux_last_chunk_on_ties": ("j = int(np.argmax(seg))                          # first maximum",
                               "j = len(seg) - 1 - int(np.argmax(seg[::-1]))"),
    "aux_grad_not_divided_by_heads": ("g = ds[i] / H", "g = ds[i]"),
    "bf16_ord_negatives_reversed": ("np.where(b & 0x8000, 0x8000 - b, b)",
                                    "np.where(b & 0x8000, b - 0x8000, b)"),
    "bf16_ord_negative_zero_apart": ("np.where(b & 0x8000, 0x8000 - b, b)",
                                     "np.where(b & 0x8000, 0x7FFF - b, b)"),
    "interleave_attends_new_tokens_only": (
        "out = sparse_attend(Q_new, state.K_loc, state.V_loc, Kbar, Vbar, doc_chunk_offsets,",
        "out = sparse_attend(Q_new, np.asarray(K_new), np.asarray(V_new), Kbar, Vbar, doc_chunk_offsets,"),
    "interleave_keys_replaced_not_appended": (
        "state.K_loc = np.concatenate([state.K_loc, np.asarray(K_new)], axis=0)",
        "state.K_loc = np.asarray(K_new)"),
    "aux_batched_key_grad_averaged": ("dK = np.sum([o[2] for o in outs], axis=0)",
                                      "dK = np.mean([o[2] for o in outs], axis=0)"),
    "aux_choice_ignored": ("            c, t = int(choice[0][i]), int(choice[1][i])",
                           "            pass"),
    "aux_choice_of_query_0_for_all": ("choice=None if choice is None else (choice[0][b], choice[1][b]))",
                                      "choice=None if choice is None else (choice[0][0], choice[1][0]))"),
    "aux_choice_keeps_free_score": ("s[i], c_star[i], t_star[i] = S[t, c], c, t",
                                    "s[i], c_star[i], t_star[i] = Sc[c], c, t"),
}

# fast pins first: the loop stops at the first pin that fails
PINS = [getattr(P, n) for n in dir(P) if n.startswith("test_")]
PINS.sort(key=lambda f: (f.__name__ in ("test_planted_recall_cfg1",
                                        "test_interleave_incremental_equals_full_reroute"),
                         f.__name__))


def _mutant(old, new):
    assert SRC.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("msa_oracle_mutant")
    mod.__file__ = "<mutant>"
    exec(compile(SRC.replace(old, new), "<mutant>", "exec"), mod.__dict__)
    return mod


def test_unmutated_oracle_passes_all_pins():
    mod = _mutant("N_Q_HEADS = 32", "N_Q_HEADS = 32")
    saved = P.O
    try:
        P.O = mod
        for pin in PINS:
            pin()
    finally:
        P.O = saved


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name):
    mod = _mutant(*MUTATIONS[name])
    saved = P.O
    caught = None
    try:
        P.O = mod
        for pin in PINS:
            try:
                pin()
            except Exception as e:  # an assertion, or the mutant breaking a shape
                caught = (pin.__name__, type(e).__name__)
                break
    finally:
        P.O = saved
    assert caught is not None, f"no pin caught mutation {name}"
