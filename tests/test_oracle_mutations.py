"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake in a copy of the oracle's source -- a swapped operand, a
wrong index, sign, bias or tie order, a dropped step -- loads the copy as a module of its own, runs
the pins that should notice, with the copy in place of the oracle, and requires that at least one
of them fails.  A mistake no pin notices would mean the oracle can be wrong without the tests
saying so.  The oracle module itself is never modified."""
import os
import types

import pytest

import test_oracle_formats as F
import test_oracle_layer as L

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "moe_oracle.py")
with open(SRC_PATH, encoding="utf-8") as fh:
    SRC = fh.read()


# name: (text in the oracle, replacement, pins expected to catch it as (module, test, args))
MUTATIONS = {
    "gate_up_swapped": ("return gu[:I], gu[I:], wd", "return gu[I:], gu[:I], wd",
                        [(L, "test_ffn_closed_form_with_permutation_weights", ("bf16",))]),
    "down_transposed": ("return ain @ wd.T", "return ain @ wd",
                        [(L, "test_ffn_closed_form_with_permutation_weights", ("f32",))]),
    "silu_sign": ("return z / (1.0 + np.exp(-z))", "return z / (1.0 + np.exp(z))",
                  [(L, "test_silu_reference_values", ())]),
    "nibble_order": ("codes[:, 0::2] = b & 0xF\n        codes[:, 1::2] = b >> 4",
                     "codes[:, 0::2] = b >> 4\n        codes[:, 1::2] = b & 0xF",
                     [(F, "test_mxfp4_nibble_order_and_scales", ())]),
    "e4m3_bias": ("np.ldexp(1.0 + m / 8.0, e - 7)", "np.ldexp(1.0 + m / 8.0, e - 8)",
                  [(F, "test_e4m3fn_all_codes_match_torch", ()), (F, "test_e4m3fn_spec_spot_values", ())]),
    "e2m1_subnormal": ("np.where(e == 0, m / 2.0,", "np.where(e == 0, m,",
                       [(F, "test_e2m1_matches_spec_table", ())]),
    "bf16_shift": ("<< np.uint32(16)", "<< np.uint32(15)", [(F, "test_bf16_matches_torch", ())]),
    "block_scale_transposed": ("sc[rows[:, None], cols[None, :]]", "sc[cols[None, :] % sc.shape[0], rows[:, None] % sc.shape[1]]",
                               [(F, "test_fp8_block_scale_indexing", ())]),
    "missing_renorm": ("return picked / picked.sum(axis=1, keepdims=True)", "return picked",
                       [(L, "test_softmax_renorm_is_softmax_of_selected_logits", ()),
                        (L, "test_sigmoid_renorm_matches_expit", ())]),
    "tie_order": ("key=lambda e: (-float(logits32[t, e]), int(e))", "key=lambda e: (-float(logits32[t, e]), -int(e))",
                  [(L, "test_select_topk_matches_lexsort", ())]),
    "sigmoid_sign": ("return 1.0 / (1.0 + np.exp(-l))", "return 1.0 / (1.0 + np.exp(l))",
                     [(L, "test_sigmoid_renorm_matches_expit", ())]),
    "unstable_permutation": ("perm.extend(np.nonzero(slot == s)[0].tolist())",
                             "perm.extend(np.nonzero(slot == s)[0][::-1].tolist())",
                             [(L, "test_permutation_matches_stable_argsort", (False,))]),
    "miss_test": ("r = np.nonzero(slot < 0)[0]", "r = np.nonzero(slot <= 0)[0]",
                  [(L, "test_permutation_matches_stable_argsort", (True,)),
                   (L, "test_compact_plus_misses_equals_all_resident", ())]),
    "miss_weight_not_full_k": ("np.asarray(topk_w, np.float64).reshape(-1)[r]", "np.ones(r.size)",
                               [(L, "test_compact_plus_misses_equals_all_resident", ())]),
    "combine_wrong_gate": ("out[t] += w[t, j] * y_perm[p]", "out[t] += w[t, (j + 1) % k] * y_perm[p]",
                           [(L, "test_layer_matches_dense_brute_force", ("bf16",))]),
    "act_quant_exponent": ("np.maximum(ex - 1 - 8, -127)", "np.maximum(ex - 1 - 7, -127)",
                           [(F, "test_act_quant_block_rule", ())]),
    "act_quant_no_e8m0_clamp": ("np.maximum(ex - 1 - 8, -127)", "ex - 1 - 8",
                                [(F, "test_act_quant_e8m0_lower_clamp", ())]),
    "e4m3_round_ties_up": ("r = np.round(mag / q) * q", "r = np.floor(mag / q + 0.5) * q",
                           [(F, "test_e4m3fn_round_matches_torch_cast", ())]),
    "plan_ties_to_larger_id": ("order = np.lexsort((np.arange(h.size), -h))", "order = np.lexsort((-np.arange(h.size), -h))",
                               [(L, "test_plan_slots_brute_force", ())]),
    "lru_most_recent_first": ("key=lambda s: (lu[s], s))", "key=lambda s: (-lu[s], s))",
                              [(L, "test_lru_refill_worked_example", ())]),
    "tiers_second_tier_dropped": ("            elif ib[t, j] >= 0:", "            elif False:",
                                  [(L, "test_two_tiers_equal_one_pool", ())]),
}


def _mutant(old, new):
    assert SRC.count(old) == 1, f"mutation anchor must occur once in the oracle: {old!r}"
    mod = types.ModuleType("moe_oracle_mutant")
    mod.__file__ = SRC_PATH
    exec(compile(SRC.replace(old, new), "moe_oracle_mutant", "exec"), mod.__dict__)
    return mod


def test_pins_pass_on_the_oracle_itself():
    # the same pins, unmutated, must pass (so that a failure below is the mutation's doing)
    for _, _, pins in MUTATIONS.values():
        for mod, name, args in pins:
            getattr(mod, name)(*args)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    old, new, pins = MUTATIONS[name]
    mutant = _mutant(old, new)
    caught = []
    for mod, test, args in pins:
        monkeypatch.setattr(mod, "O", mutant)
        try:
            getattr(mod, test)(*args)
        except Exception as e:  # an assertion, or the mistake breaking the computation outright
            caught.append(f"{test}: {type(e).__name__}")
        finally:
            monkeypatch.undo()
    assert caught, f"no pin noticed the planted mistake {name!r}"
