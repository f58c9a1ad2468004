"""The oracle's pins must catch plausible mistakes in the oracle.

Each case below plants one slip in a copy of an oracle function, on the CPU:
- a dropped or sign-flipped term;
- a transposed operand;
- the read-out taken before the write;
- a wrong head map;
- a misplaced scale;
- a strict/inclusive mask swapped;
- a wrong slot rule.

The copy is made from the function's own source with one textual
replacement, and stands in for the original while the pins of
test_oracle_pins.py run. A case passes when at least one pin fails on the
mutant. The unmutated oracle must pass every pin of the same list, which the
control case checks, so a failure is the mutant's doing.

Mutants that cannot change a result on the tables the library accepts are
not listed. For example, reading a source from the pool as updated so far
equals reading it as it was on entry: a validated table lets no destination
be another entry's source.
"""

import importlib.util
import inspect
import os

import pytest

import oracle
import oracle.gdn_oracle as G

_PINS_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "test_oracle_pins.py")


def _load_pins():
    spec = importlib.util.spec_from_file_location("_oracle_pins_for_mutants", _PINS_PATH)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


P = _load_pins()

# (pin, arguments): one instance of each pin, sized small
PINS = [
    (P.test_hand_worked_two_tokens, ()),
    (P.test_l2_normalize_with_eps_by_hand, ()),
    (P.test_beta0_g0_leaves_state_and_reads_it, (8, 24)),
    (P.test_unit_key_full_write_reads_back_v, (8, 24)),
    (P.test_delta_write_is_fixed_on_k_and_its_complement, (0,)),
    (P.test_pure_decay_closed_form, ()),
    (P.test_associative_memory_with_basis_keys, ()),
    (P.test_full_write_is_idempotent, ()),
    (P.test_linear_in_initial_state_and_values, ()),
    (P.test_value_columns_are_independent, ()),
    (P.test_value_head_reads_key_head_h_div_group, ()),
    (P.test_query_and_key_scale_invariance_and_output_scale, ()),
    (P.test_chunk_form_equals_token_loop, (16, 65)),
    (P.test_chunk_form_equals_token_loop, (4, 130)),
    (P.test_prefill_slot_semantics, ()),
    (P.test_decode_steps_in_place_equal_one_sequence, ()),
    (P.test_decode_step_matches_prefill_rows, ()),
    (P.test_prefill_checkpoints_equal_chunk_form_of_each_prefix, ()),
    (P.test_verify_states_equal_chunk_form_of_each_prefix, ()),
    (P.test_verify_lengths_skips_and_unstored_positions, ()),
    (P.test_verify_in_place_first_position_reads_original, ()),
    (P.test_pack_unpack_round_trip_and_edge_entries, ()),
    (P.test_slot_model_alloc_lowest_first_all_or_nothing, ()),
    (P.test_slot_model_refcounts_and_cow, ()),
    (P.test_slot_model_validate, ()),
]

# (id, oracle object, text in its source, replacement)
MUTANTS = [
    # the token rule
    ("decay_dropped", "gated_delta_token", "S = np.exp(g) * S", "S = S"),
    ("decay_sign", "gated_delta_token", "S = np.exp(g) * S", "S = np.exp(-g) * S"),
    ("delta_sign", "gated_delta_token", "(np.asarray(v, np.float64) - Sk)", "(np.asarray(v, np.float64) + Sk)"),
    ("beta_dropped", "gated_delta_token", "delta = beta * (", "delta = ("),
    ("beta_squared", "gated_delta_token", "delta = beta * (", "delta = beta * beta * ("),
    ("readout_before_write", "gated_delta_token", 'o = np.einsum("...ij,...j->...i", S, qt)',
     'o = np.einsum("...ij,...j->...i", S - delta[..., :, None] * kh[..., None, :], qt)'),
    ("readout_transposed", "gated_delta_token", 'o = np.einsum("...ij,...j->...i", S, qt)',
     'o = np.einsum("...ji,...j->...i", S, qt) if S.shape[-1] == S.shape[-2] else '
     'np.einsum("...ij,...j->...i", S, qt)'),
    ("recall_transposed", "gated_delta_token", 'Sk = np.einsum("...ij,...j->...i", S, kh)',
     'Sk = np.einsum("...ji,...j->...i", S, kh) if S.shape[-1] == S.shape[-2] else '
     'np.einsum("...ij,...j->...i", S, kh)'),
    ("scale_on_k", "gated_delta_token", "kh = l2_normalize(k, eps)\n    qt = l2_normalize(q, eps) * scale",
     "kh = l2_normalize(k, eps) * scale\n    qt = l2_normalize(q, eps)"),
    ("scale_dropped", "gated_delta_token", "qt = l2_normalize(q, eps) * scale", "qt = l2_normalize(q, eps)"),
    ("k_not_normalised", "gated_delta_token", "kh = l2_normalize(k, eps)", "kh = np.asarray(k, np.float64)"),
    ("q_not_normalised", "gated_delta_token", "qt = l2_normalize(q, eps) * scale",
     "qt = np.asarray(q, np.float64) * scale"),
    # normalisation
    ("eps_sign", "l2_normalize", "keepdims=True) + eps)", "keepdims=True) - eps)"),
    ("norm_without_sqrt", "l2_normalize", "np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)",
     "(np.sum(x * x, axis=-1, keepdims=True) + eps)"),
    # head map
    ("head_map_interleaved", "_head_map", "np.arange(HV) // (HV // HK)", "np.arange(HV) % HK"),
    # storage orientation of the token loop
    ("state_not_transposed_back", "recurrent_sequence", "return o, np.transpose(S, (0, 2, 1)).copy()",
     "return o, (np.transpose(S, (0, 2, 1)) if S.shape[-1] != S.shape[-2] else S).copy()"),
    # chunk form
    ("chunk_decay_difference_sign", "chunked_sequence", "diff = gam[:, None] - gam[None, :]",
     "diff = gam[None, :] - gam[:, None]"),
    ("chunk_A_mask_inclusive", "chunked_sequence", "A = np.where(tri_strict,", "A = np.where(tri_incl,"),
    ("chunk_P_mask_strict", "chunked_sequence", "P = np.where(tri_incl,", "P = np.where(tri_strict,"),
    ("chunk_inter_output_dropped", "chunked_sequence", "np.exp(gam)[:, None] * (Qt @ H[h]) + P @ U", "P @ U"),
    ("chunk_inter_output_undecayed", "chunked_sequence", "np.exp(gam)[:, None] * (Qt @ H[h]) + P @ U",
     "(Qt @ H[h]) + P @ U"),
    ("chunk_W_decay_dropped", "chunked_sequence", "(b * np.exp(gam))[:, None] * Kh", "b[:, None] * Kh"),
    ("chunk_U_sign", "chunked_sequence", "U = Up - W @ H[h]", "U = Up + W @ H[h]"),
    ("chunk_advance_key_decay_dropped", "chunked_sequence", "Kd = np.exp(gam[-1] - gam)[:, None] * Kh",
     "Kd = Kh"),
    ("chunk_advance_state_decay_dropped", "chunked_sequence", "H[h] = np.exp(gam[-1]) * H[h] + Kd.T @ U",
     "H[h] = H[h] + Kd.T @ U"),
    ("chunk_solve_sign", "chunked_sequence", "np.linalg.solve(np.eye(c) + A, np.eye(c))",
     "np.linalg.solve(np.eye(c) - A, np.eye(c))"),
    # slot semantics of prefill
    ("negative_src_reads_last_slot", "prefill", "if src[n] >= 0:", "if src[n] >= -1:"),
    ("skipped_rows_written", "prefill", "if dst[n] < 0:\n            continue", "if dst[n] < -1:\n            continue"),
    ("in_place_entry_not_stored", "prefill", "new_pool[dst[n]] = Hn.astype(np.float32)",
     "new_pool[dst[n]] = Hn.astype(np.float32) if dst[n] != src[n] else new_pool[dst[n]]"),
    ("empty_sequence_zeroed", "prefill", "Hn = H0.copy()", "Hn = np.zeros_like(H0)"),
    ("checkpoint_taken_before_its_chunk", "prefill",
     "o[s_:e_], Hn = run(Hn, s_, e_)\n"
     "                    if ckpt[c0 + j] >= 0:\n"
     "                        stored[c0 + j] = Hn.copy()",
     "if ckpt[c0 + j] >= 0:\n"
     "                        stored[c0 + j] = Hn.copy()\n"
     "                    o[s_:e_], Hn = run(Hn, s_, e_)"),
    # slot model
    ("alloc_highest_first", "SlotPoolModel", "out = free[:n]", "out = free[::-1][:n]"),
    ("alloc_partial", "SlotPoolModel", "if len(free) < n:\n            return GDN_E_NO_SLOTS, []",
     "if not free and n:\n            return GDN_E_NO_SLOTS, []"),
    ("cow_always_in_place", "SlotPoolModel", "if src >= 0 and self.ref[src] == 1:",
     "if src >= 0 and self.ref[src] >= 1:"),
    ("release_below_zero", "SlotPoolModel", "if self.ref[slot] == 0:\n            return GDN_E_SLOT_STATE\n"
     "        self.ref[slot] -= 1", "self.ref[slot] = max(self.ref[slot] - 1, 0)"),
]


def _mutant(name, old, new):
    obj = getattr(G, name)
    src = inspect.getsource(obj)
    assert src.count(old) == 1, f"{name}: the text to replace must occur exactly once"
    ns = dict(vars(G))
    exec(compile(src.replace(old, new), f"<mutant of {name}>", "exec"), ns)
    return ns[name]


def _patch(monkeypatch, name, value):
    for mod in (G, oracle, P):
        if hasattr(mod, name):
            monkeypatch.setattr(mod, name, value)


def _failing_pins():
    failed = []
    for pin, args in PINS:
        try:
            pin(*args)
        except Exception as e:                  # an exception is a failed pin as well
            failed.append((pin.__name__, type(e).__name__))
    return failed


def test_unmutated_oracle_passes_every_listed_pin():
    assert _failing_pins() == []


@pytest.mark.parametrize("mid,name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(monkeypatch, mid, name, old, new):
    _patch(monkeypatch, name, _mutant(name, old, new))
    failed = _failing_pins()
    assert failed, f"mutant {mid} of {name} passes every pin"
