"""Pins of the oracle's routing variants (fixed top-k, clamped Top-p count, local window),
plus planted mistakes that the pins must catch.

Sources: the FVAttn summary (Top-p routing paragraph contrasts Top-p with a fixed Top-k) and
the tutorial's block-sparse section 5.2 (top-k key blocks by pooled score, plus a local
window of neighbouring blocks kept as a floor).
"""
import itertools
import math

import numpy as np
import pytest

import oracle
import oracle.topp_oracle as T


def _uniform_case(nb=16, block=64, d=32):
    """k == 0 gives equal pooled scores, so every importance is 1/nkb exactly."""
    N = nb * block
    rng = np.random.default_rng(5)
    q = rng.standard_normal((N, d))
    k = np.zeros((N, d))
    return q, k, N, block


def _kept(q, k, bq, bk, **kw):
    kept, _ = oracle.route_head(q, k, bq, bk, kw.pop("p", 0.9), **kw)
    return [set(map(int, x)) for x in kept]


# ---- fixed top-k -------------------------------------------------------------------------
@pytest.mark.parametrize("kk", [1, 5, 16, 40])
def test_topk_uniform_keeps_lowest_indices(kk):
    """All importances tie, so top-k is the k lowest block indices (tie rule)."""
    q, k, N, b = _uniform_case()
    for row in _kept(q, k, b, b, mode="topk", topk=kk):
        assert row == set(range(min(kk, 16)))


def test_topk_one_hot():
    """One key block scores far above the others (which tie): it is kept, then the lowest
    other indices fill the remaining k - 1 places."""
    nb, b, d = 12, 32, 16
    N = nb * b
    q = np.ones((N, d))
    k = np.zeros((N, d))
    k[7 * b:8 * b] = 5.0
    for row in _kept(q, k, b, b, mode="topk", topk=4):
        assert row == {7, 0, 1, 2}


def test_topk_bruteforce_maximum_mass():
    """On random inputs the kept k blocks carry the maximum mass of any k-subset."""
    rng = np.random.default_rng(11)
    nb, b, d = 10, 16, 8
    N = nb * b - 5                      # ragged last block
    q = rng.standard_normal((N, d)) * 2
    k = rng.standard_normal((N, d)) * 2
    P = oracle.block_importance(oracle.block_scores(oracle.pool_blocks(q, b), oracle.pool_blocks(k, b)))
    for kk in (1, 3, 6):
        kept = _kept(q, k, b, b, mode="topk", topk=kk)
        for i, row in enumerate(kept):
            assert len(row) == kk
            best = max(sum(P[i, list(s)]) for s in itertools.combinations(range(nb), kk))
            assert math.isclose(sum(P[i, list(row)]), best, rel_tol=0, abs_tol=1e-15)


def test_topk_with_window_matches_tutorial_construction():
    """The tutorial's construction, restated: block means of q and k (no padding: N is a
    multiple of the block), scores qbar kbar^T / sqrt(d), the top-k key blocks of each query
    block, then blocks i-w .. i+w added.  Scores here are distinct, so the set is unique."""
    rng = np.random.default_rng(23)
    b, nb, d, kk, w = 16, 12, 8, 3, 2
    N = nb * b
    q = rng.standard_normal((N, d))
    k = rng.standard_normal((N, d))
    qb = q.reshape(nb, b, d).mean(axis=1)
    kb = k.reshape(nb, b, d).mean(axis=1)
    sc = qb @ kb.T / math.sqrt(d)
    assert len(np.unique(sc)) == sc.size
    mask = np.zeros((nb, nb), dtype=bool)
    top = np.argsort(-sc, axis=1)[:, :kk]
    for i in range(nb):
        mask[i, top[i]] = True
        for off in range(-w, w + 1):
            if 0 <= i + off < nb:
                mask[i, i + off] = True
    ref = [set(map(int, np.nonzero(mask[i])[0])) for i in range(nb)]
    assert _kept(q, k, b, b, mode="topk", topk=kk, window=w) == ref


# ---- clamped Top-p count -----------------------------------------------------------------
@pytest.mark.parametrize("kmin,kmax,expect", [(1, 0, 8), (1, 5, 5), (10, 0, 10), (20, 0, 16), (8, 8, 8)])
def test_clamp_uniform(kmin, kmax, expect):
    """Uniform importance over 16 blocks: Top-p at p = 0.5 keeps exactly 8 (dyadic sums);
    the clamp moves the count and the kept set stays the lowest indices."""
    q, k, N, b = _uniform_case()
    for row in _kept(q, k, b, b, p=0.5, k_min=kmin, k_max=kmax):
        assert row == set(range(expect))


def test_clamp_equal_bounds_is_topk():
    rng = np.random.default_rng(3)
    N, b, d = 700, 32, 16
    q = rng.standard_normal((N, d)) * 2
    k = rng.standard_normal((N, d)) * 2
    assert _kept(q, k, b, b, p=0.7, k_min=5, k_max=5) == _kept(q, k, b, b, mode="topk", topk=5)


# ---- local window ------------------------------------------------------------------------
def test_window_equal_blocks():
    """Equal block sizes: the window is i-w .. i+w, clipped to the sequence."""
    q, k, N, b = _uniform_case()
    kept = _kept(q, k, b, b, p=0.5, window=2)
    base = set(range(8))
    assert kept[12] == base | {10, 11, 12, 13, 14}
    assert kept[15] == base | {13, 14, 15}
    assert kept[0] == base


def test_window_follows_token_span():
    """Query blocks of 128 tokens over key blocks of 64: query block i spans key blocks 2i and
    2i+1, so a window of 1 forces 2i-1 .. 2i+2."""
    N = 16 * 64
    for i, expect in [(0, [0, 1, 2]), (3, [5, 6, 7, 8]), (7, [13, 14, 15])]:
        assert list(oracle.window_blocks(i, N, 128, 64, 1)) == expect
    # query blocks of 32 tokens over key blocks of 64: block 5 (tokens 160..191) sits in key
    # block 2, so a window of 2 forces 0 .. 4
    assert list(oracle.window_blocks(5, N, 32, 64, 2)) == [0, 1, 2, 3, 4]
    # ragged tail: N = 1000, key blocks of 64 (16 blocks, the last one short)
    assert list(oracle.window_blocks(15, 1000, 64, 64, 3)) == [12, 13, 14, 15]
    assert list(oracle.window_blocks(4, N, 64, 64, 0)) == []


# ---- planted mistakes --------------------------------------------------------------------
_ORIG_SEL = T.selection_count
_ORIG_WIN = T.window_blocks


def _win_plus_one(i, n, bq, bk, w):
    return _ORIG_WIN(i, n, bq, bk, w + 1 if w > 0 else 0)


def _win_on_index(i, n, bq, bk, w):       # centred on block index i instead of the token span
    if w <= 0:
        return np.zeros(0, dtype=np.int64)
    nkb = -(-n // bk)
    return np.arange(max(0, i - w), min(nkb - 1, i + w) + 1, dtype=np.int64)


def _sel_topk_plus_one(Ps, mode="topp", p=0.9, topk=0, k_min=1, k_max=0):
    c = _ORIG_SEL(Ps, mode, p, topk, k_min, k_max)
    return min(c + 1, Ps.shape[0]) if mode == "topk" else c


def _sel_no_kmax(Ps, mode="topp", p=0.9, topk=0, k_min=1, k_max=0):
    return _ORIG_SEL(Ps, mode, p, topk, k_min, 0)


def _sel_no_kmin(Ps, mode="topp", p=0.9, topk=0, k_min=1, k_max=0):
    return _ORIG_SEL(Ps, mode, p, topk, 1, k_max)


def _order_ties_high(P):
    n = P.shape[-1]
    return (n - 1 - np.argsort(-P[..., ::-1], axis=-1, kind="stable"))


MUTANTS = {
    "window_one_too_wide": ("window_blocks", _win_plus_one),
    "window_on_block_index": ("window_blocks", _win_on_index),
    "topk_one_too_many": ("selection_count", _sel_topk_plus_one),
    "clamp_ignores_kmax": ("selection_count", _sel_no_kmax),
    "clamp_ignores_kmin": ("selection_count", _sel_no_kmin),
    "ties_to_higher_index": ("routing_order", _order_ties_high),
}

_PINS = [
    (test_topk_uniform_keeps_lowest_indices, 5),
    (test_topk_one_hot,),
    (test_topk_bruteforce_maximum_mass,),
    (test_topk_with_window_matches_tutorial_construction,),
    (test_clamp_uniform, 1, 5, 5),
    (test_clamp_uniform, 10, 0, 10),
    (test_window_equal_blocks,),
    (test_window_follows_token_span,),
]


def _caught():
    for pin in _PINS:
        try:
            pin[0](*pin[1:])
        except AssertionError:
            return True
    return False


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_variant_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(T, attr, fn)
    if hasattr(oracle, attr):
        monkeypatch.setattr(oracle, attr, fn)
    assert _caught(), f"no pin detects mutant {name}"


def test_unmutated_variants_pass():
    assert not _caught()
