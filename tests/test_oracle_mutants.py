"""Plant plausible mistakes in the oracle (on the CPU, via monkeypatch) and check
that at least one pin in test_oracle_pins catches each of them."""
import math

import numpy as np
import pytest

import oracle
import oracle.topp_oracle as T
import test_oracle_pins as pins

GOLD = pins.GOLD
_ORIG_COUNT = T.topp_count


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def _all_pins():
    out = []
    for c in GOLD["uniform_importance"]["cases"]:
        out.append((pins.test_uniform_importance_dyadic, c))
    for c in GOLD["two_block_logistic"]["cases"]:
        out.append((pins.test_two_block_scale, c))
    for c in GOLD["tie_rule"]["cases"]:
        out.append((pins.test_tie_rule_lower_index, c))
    for f in (pins.test_pool_ragged_mean_closed_form, pins.test_short_sequence_single_block_always_kept,
              pins.test_one_hot_block_keeps_one,
              pins.test_bruteforce_minimality_random_ragged, pins.test_zero_keys_average_kept_values,
              pins.test_single_token_block_returns_its_value, pins.test_sparse_equals_masked_sdpa,
              pins.test_dense_gate_full_coverage):
        out.append((f,))
    return out


def _caught():
    return any(_fails(*p) for p in _all_pins())


MUTANTS = {
    "no_sqrt_d_scale": ("block_scores", lambda qb, kb: qb @ kb.T),
    "scale_1_over_d": ("block_scores", lambda qb, kb: (qb @ kb.T) / qb.shape[1]),
    "ascending_order": ("routing_order", lambda P: np.argsort(P, axis=-1, kind="stable")),
    "ties_to_higher_index": ("routing_order",
                             lambda P: (P.shape[-1] - 1) - np.argsort(-P[..., ::-1], axis=-1, kind="stable")),
    "strict_greater_cut": ("topp_count", lambda Ps, p: (len(Ps) if p >= 1 else
                           (int(np.nonzero(np.cumsum(Ps) > p)[0][0]) + 1
                            if np.any(np.cumsum(Ps) > p) else len(Ps)))),
    "one_block_too_many": ("topp_count", lambda Ps, p: min(len(Ps), _ORIG_COUNT(Ps, p) + 1)),
    "padded_mean": ("pool_blocks", lambda x, b: np.stack([
        np.asarray(x, np.float64)[s:e].sum(0) / b for s, e in T.block_bounds(x.shape[0], b)])),
    "no_softmax_max_shift_but_sum_norm_of_scores": ("block_importance",
                                                     lambda s: np.maximum(s, 1e-300) / np.maximum(s, 1e-300).sum(-1, keepdims=True)),
    "attention_no_scale": ("_attend", lambda qr, ks, vs: (lambda w: (w @ vs) / w.sum(1, keepdims=True))(
        np.exp(qr @ ks.T - (qr @ ks.T).max(1, keepdims=True)))),
    "attention_transposed_values": ("_attend", lambda qr, ks, vs: (lambda s: (np.exp(s - s.max(1, keepdims=True)) @ ks)
                                    / np.exp(s - s.max(1, keepdims=True)).sum(1, keepdims=True))(
        qr @ ks.T / math.sqrt(qr.shape[1]))),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(T, attr, fn)
    if hasattr(oracle, attr):
        monkeypatch.setattr(oracle, attr, fn)
    assert _caught(), f"no pin detects mutant {name}"


def test_unmutated_oracle_passes_all_pins():
    assert not _caught()
