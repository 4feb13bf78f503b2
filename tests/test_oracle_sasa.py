"""Pins of the oracle's SASA step (FVAttn summary, SASA section: ranks with slack before the
synchronisation point add the highest-importance blocks that Top-p left out, within their
slack, scaled by an augmentation coefficient and gated by a trigger threshold), plus planted
mistakes that the pins must catch."""
import math

import numpy as np
import pytest

import oracle
import oracle.topp_oracle as T


def _two_heads(nb=16, b=32, d=16):
    """Head 0: key block 7 scores far above the others, which all tie (Top-p keeps only
    block 7).  Head 1: k == 0, every importance 1/nb (Top-p at p = 0.5 keeps 0..7)."""
    N = nb * b
    q = np.ones((1, 2, N, d))
    k = np.zeros((1, 2, N, d))
    k[0, 0, 7 * b:8 * b] = 3.0
    return q, k, b


def test_closed_form_two_heads():
    q, k, b = _two_heads()
    r = oracle.route_sasa(q, k, b, b, 0.5, groups=2, alpha=0.5, tau=0.0)
    assert [len(x) for x in r["base_kept"][0]] == [1] * 16
    assert [len(x) for x in r["base_kept"][1]] == [8] * 16
    assert r["critical"] == 128 and r["budgets"] == [56, 0]
    # the 15 candidates of every head-0 row tie: rows 0, 1, 2 take all, row 3 takes 11
    full = list(range(16))
    for i in range(3):
        assert list(r["kept"][0][i]) == full
    assert list(r["kept"][0][3]) == [0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11]
    for i in range(4, 16):
        assert list(r["kept"][0][i]) == [7]
    for i in range(16):
        assert list(r["kept"][1][i]) == list(range(8))
    assert r["head_load"].tolist() == [72, 128]


@pytest.mark.parametrize("alpha,tau,expect0", [(0.0, 0.0, 0), (1.0, 0.0, 112), (0.5, 0.9, 0),
                                               (0.5, 0.87, 56), (0.25, 0.0, 28), (0.3, 0.0, 33)])
def test_coefficient_and_trigger(alpha, tau, expect0):
    """slack / critical = 112 / 128 = 0.875: a trigger of 0.9 blocks the augmentation, 0.87
    lets it through; the budget is floor(alpha * slack)."""
    q, k, b = _two_heads()
    r = oracle.route_sasa(q, k, b, b, 0.5, groups=2, alpha=alpha, tau=tau)
    assert r["budgets"][0] == expect0
    assert r["head_load"][0] == 16 + expect0


def test_given_critical_path():
    """A critical path above every group's load gives every group slack."""
    q, k, b = _two_heads()
    r = oracle.route_sasa(q, k, b, b, 0.5, groups=2, alpha=1.0, tau=0.0, critical=160)
    assert r["budgets"] == [144, 32]
    assert r["head_load"].tolist() == [160, 160]


def _random_case(seed, H=4, N=700, b=32, d=16):
    rng = np.random.default_rng(seed)
    alphas = rng.uniform(0.0, 3.0, H)
    q = rng.standard_normal((1, H, N, d)) + alphas[None, :, None, None] * np.sin(np.arange(N))[None, None, :, None]
    k = rng.standard_normal((1, H, N, d)) * (1 + alphas[None, :, None, None])
    return q, k, b


@pytest.mark.parametrize("seed,groups,alpha,tau", [(1, 2, 0.5, 0.0), (2, 4, 0.8, 0.05), (3, 2, 1.0, 0.0)])
def test_invariants_random(seed, groups, alpha, tau):
    q, k, b = _random_case(seed)
    r = oracle.route_sasa(q, k, b, b, 0.8, groups=groups, alpha=alpha, tau=tau)
    H = q.shape[1]
    grp = [h * groups // H for h in range(H)]
    base = [sum(len(x) for x in r["base_kept"][h]) for h in range(H)]
    L = [sum(base[h] for h in range(H) if grp[h] == g) for g in range(groups)]
    crit = max(L)
    assert r["critical"] == crit
    for g in range(groups):
        hs = [h for h in range(H) if grp[h] == g]
        added, rest = [], []
        for h in hs:
            P = r["P"][h]
            for i, (b0, b1) in enumerate(zip(r["base_kept"][h], r["kept"][h])):
                assert set(b0) <= set(b1)
                for j in range(P.shape[1]):
                    if j in b1 and j not in b0:
                        added.append(P[i, j])
                    elif j not in b1:
                        rest.append(P[i, j])
        slack = crit - L[g]
        want = int(math.floor(alpha * slack)) if (slack > 0 and slack >= tau * crit) else 0
        assert len(added) == min(want, len(added) + len(rest))
        assert L[g] + len(added) <= crit
        if added and rest:
            assert min(added) >= max(rest)


# ---- planted mistakes --------------------------------------------------------------------
_ORIG = T.sasa_augment


def _ties_high_row(kept, P, groups, alpha, tau, critical=0):
    """Reverse the row order of the heads before selecting, so ties go to higher rows."""
    flipped_kept = [head[::-1] for head in kept]
    flipped_P = [p[::-1] for p in P]
    out, b, c = _ORIG(flipped_kept, flipped_P, groups, alpha, tau, critical)
    return [head[::-1] for head in out], b, c


_ORIG_BUDGET = T.sasa_budget


def _budget_ignore_tau(slack, critical, alpha, tau):
    return _ORIG_BUDGET(slack, critical, alpha, 0.0)


def _budget_ceil(slack, critical, alpha, tau):
    if slack <= 0 or slack < tau * critical:
        return 0
    return int(math.ceil(alpha * slack))


def _per_row_round_robin(kept, P, groups, alpha, tau, critical=0):
    """Budget spread evenly over rows instead of the highest importance across the group."""
    out, budgets, crit = _ORIG(kept, P, groups, 0.0, tau, critical)
    H = len(kept)
    nqb, nkb = P[0].shape
    for g, bud in enumerate(_ORIG(kept, P, groups, alpha, tau, critical)[1]):
        hs = [h for h in range(H) if h * groups // H == g]
        rows = [(h, i) for h in hs for i in range(nqb)]
        n = 0
        while n < bud:
            progressed = False
            for h, i in rows:
                if n >= bud:
                    break
                rest = [j for j in np.argsort(-P[h][i], kind="stable") if j not in out[h][i]]
                if rest:
                    out[h][i] = np.union1d(out[h][i], [rest[0]]).astype(np.int64)
                    n += 1
                    progressed = True
            if not progressed:
                break
    return out, budgets, crit


def _critical_is_mean(kept, P, groups, alpha, tau, critical=0):
    H = len(kept)
    loads = [sum(len(x) for x in kept[h]) for h in range(H)]
    L = [sum(loads[h] for h in range(H) if h * groups // H == g) for g in range(groups)]
    return _ORIG(kept, P, groups, alpha, tau, critical or int(np.mean(L)))


MUTANTS = {
    "ties_to_higher_row": ("sasa_augment", _ties_high_row),
    "trigger_ignored": ("sasa_budget", _budget_ignore_tau),
    "budget_rounded_up": ("sasa_budget", _budget_ceil),
    "round_robin_over_rows": ("sasa_augment", _per_row_round_robin),
    "critical_path_is_mean": ("sasa_augment", _critical_is_mean),
}

_PINS = [
    (test_closed_form_two_heads,),
    (test_coefficient_and_trigger, 0.5, 0.9, 0),
    (test_coefficient_and_trigger, 0.25, 0.0, 28),
    (test_coefficient_and_trigger, 0.3, 0.0, 33),
    (test_given_critical_path,),
    (test_invariants_random, 1, 2, 0.5, 0.0),
]


def _caught():
    for pin in _PINS:
        try:
            pin[0](*pin[1:])
        except AssertionError:
            return True
    return False


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_sasa_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(T, attr, fn)
    monkeypatch.setattr(oracle, attr, fn)
    assert _caught(), f"no pin detects mutant {name}"


def test_unmutated_sasa_passes():
    assert not _caught()
