"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Nothing here re-types the oracle's formulas: expectations come from hand-derived
closed forms (tests/golden/closed_forms.json), brute force over every block
subset, a library routine (torch's scaled_dot_product_attention in fp64 on the
CPU) and invariants of the Top-p definition.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")))


def _route1(q_h, k_h, bq, bk, p):
    kept, extra = oracle.route_head(q_h, k_h, bq, bk, p, diagnostics=True)
    return kept, extra


# ---------------------------------------------------------------- pooling
def test_pool_ragged_mean_closed_form():
    g = GOLD["ragged_mean"]
    N, d, b = g["N"], g["d"], g["block"]
    x = np.arange(N, dtype=np.float64)[:, None] + np.arange(d)[None, :]
    pooled = oracle.pool_blocks(x, b)
    assert pooled.shape == (16, d)
    np.testing.assert_array_equal(pooled[-1], g["expected_last_block"])
    np.testing.assert_array_equal(pooled[0], g["expected_first_block"])


def test_pool_constant_blocks():
    rng = np.random.default_rng(0)
    consts = rng.standard_normal((5, 7))
    x = np.repeat(consts, [32, 32, 32, 32, 3], axis=0)  # N = 131, block 32, last block 3 tokens
    np.testing.assert_allclose(oracle.pool_blocks(x, 32), consts, rtol=0, atol=1e-15)


def test_short_sequence_single_block_always_kept():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((40, 8))
    k = rng.standard_normal((40, 8))
    kept, extra = _route1(q, k, 64, 64, 0.5)
    assert len(kept) == 1 and kept[0].tolist() == [0]
    np.testing.assert_allclose(extra["qbar"][0], q.mean(0), atol=1e-15)


# ---------------------------------------------------------------- routing closed forms
@pytest.mark.parametrize("case", GOLD["uniform_importance"]["cases"], ids=lambda c: f"p{c['p']}")
def test_uniform_importance_dyadic(case):
    g = GOLD["uniform_importance"]
    rng = np.random.default_rng(2)
    q = rng.standard_normal((g["N"], g["d"]))
    k = np.zeros((g["N"], g["d"]))
    kept, extra = _route1(q, k, g["block_q"], g["block_k"], case["p"])
    for row in kept:
        assert row.tolist() == case["kept"]
    assert (extra["counts"] == case["count"]).all()


@pytest.mark.parametrize("case", GOLD["two_block_logistic"]["cases"], ids=lambda c: f"p{c['p']}")
def test_two_block_scale(case):
    g = GOLD["two_block_logistic"]
    d = g["d"]
    q = np.zeros((g["N"], d)); q[:, 0] = 1.0
    k = np.zeros((g["N"], d)); k[:4, 0] = 2.0 * math.log(9.0)
    kept, _ = _route1(q, k, g["block_q"], g["block_k"], case["p"])
    for row in kept:
        assert row.tolist() == case["kept"]


@pytest.mark.parametrize("case", GOLD["tie_rule"]["cases"], ids=lambda c: f"p{c['p']}")
def test_tie_rule_lower_index(case):
    g = GOLD["tie_rule"]
    d = g["d"]
    q = np.zeros((g["N"], d)); q[:, 0] = 1.0
    k = np.zeros((g["N"], d))
    # blocks of 2 tokens; blocks 1 and 3 get pooled first component 2 ln 4 -> score ln 4
    k[2:4, 0] = 2.0 * math.log(4.0)
    k[6:8, 0] = 2.0 * math.log(4.0)
    kept, extra = _route1(q, k, g["block_q"], g["block_k"], case["p"])
    assert kept[0].tolist() == case["kept"]
    assert extra["order"][0].tolist() == [1, 3, 0, 2]


def test_one_hot_block_keeps_one():
    rng = np.random.default_rng(3)
    N, d = 512, 16
    q = rng.standard_normal((N, d)) * 0.1
    q[:, 0] += 1.0
    k = rng.standard_normal((N, d)) * 0.1
    k[5 * 64:6 * 64, 0] += 200.0          # key block 5 dominates every query block
    kept, extra = _route1(q, k, 64, 64, 0.9)
    assert all(r.tolist() == [5] for r in kept)


# ---------------------------------------------------------------- brute force minimality
def _bruteforce_check(P, p, kept_row, margin=1e-12):
    nb = P.shape[0]
    masks = np.array(list(itertools.product([0, 1], repeat=nb)), dtype=np.float64)
    mass = masks @ P
    size = masks.sum(1)
    if np.any(np.abs(mass - p) < margin):
        return "ambiguous"
    feasible = mass >= p
    kmin = int(size[feasible].min()) if feasible.any() else nb
    assert len(kept_row) == kmin, (len(kept_row), kmin)
    m_kept = P[kept_row].sum()
    best = mass[size == kmin].max()
    assert abs(m_kept - best) <= 1e-12
    assert m_kept >= p - 1e-15 or len(kept_row) == nb
    # the best set one smaller never reaches p
    if kmin > 1:
        assert mass[size == kmin - 1].max() < p
    return "ok"


def test_bruteforce_minimality_tiny_workload():
    w = workloads.get("tiny_f32_n1024")
    q, k = workloads.make_qkv(w, which=(0, 1))
    checked = 0
    for p in (0.5, 0.8, 0.9, 0.95):
        for h in range(w.H):
            kept, extra = _route1(q[0, h], k[0, h], w.block_q, w.block_k, p)
            for i, row in enumerate(kept):
                if _bruteforce_check(extra["P"][i], p, row) == "ok":
                    checked += 1
    assert checked >= 120


def test_bruteforce_minimality_random_ragged():
    rng = np.random.default_rng(4)
    checked = 0
    for trial in range(6):
        N = int(rng.integers(200, 330))       # 32-token key blocks: 7..11 blocks, ragged tail
        d = 8
        scale = float(rng.uniform(0.5, 6.0))
        q = rng.standard_normal((N, d)) + scale * np.sin(np.arange(N)[:, None] * 0.05 + np.arange(d))
        k = rng.standard_normal((N, d)) + scale * np.sin(np.arange(N)[:, None] * 0.05 + np.arange(d))
        p = float(rng.uniform(0.3, 0.99))
        kept, extra = _route1(q, k, 64, 32, p)
        for i, row in enumerate(kept):
            if _bruteforce_check(extra["P"][i], p, row) == "ok":
                checked += 1
    assert checked > 20


# ---------------------------------------------------------------- invariants
def test_nesting_and_loads():
    w = workloads.small_case(H=3, N=2000, d=32, block_q=64, block_k=32, seed=7,
                             alpha=("uniform", 0.0, 4.0), dtype="f32", grid=(5, 20, 20))
    q, k = workloads.make_qkv(w, which=(0, 1))
    a = oracle.route(q, k, w.block_q, w.block_k, 0.90)
    b = oracle.route(q, k, w.block_q, w.block_k, 0.95)
    for ka, kb in zip(a["kept"], b["kept"]):
        for ra, rb in zip(ka, kb):
            assert set(ra.tolist()) <= set(rb.tolist())
    for r in (a, b):
        assert r["head_load"].sum() == r["nnz"] == r["row_ptr"][-1]
        assert np.all(np.diff(r["row_ptr"]) >= 1)
        for s, e in zip(r["row_ptr"][:-1], r["row_ptr"][1:]):
            assert np.all(np.diff(r["col_idx"][s:e]) > 0)


def test_p_one_keeps_everything():
    w = workloads.get("tiny_f32_n1024")
    q, k = workloads.make_qkv(w, which=(0, 1))
    r = oracle.route(q, k, w.block_q, w.block_k, 1.0)
    assert r["nnz"] == w.rows * w.nkb


def test_lpt_worklist_invariants():
    rng = np.random.default_rng(5)
    counts = rng.integers(1, 20, size=500)
    row_ptr = np.concatenate([[0], np.cumsum(counts)])
    wl = oracle.lpt_worklist(row_ptr)
    assert sorted(wl.tolist()) == list(range(500))
    c = counts[wl]
    assert np.all(np.diff(c) <= 0)
    for a, b in zip(wl[:-1], wl[1:]):
        if counts[a] == counts[b]:
            assert a < b
    # against a plain Python sort by (-count, row)
    assert wl.tolist() == sorted(range(500), key=lambda r: (-counts[r], r))


# ---------------------------------------------------------------- attention
def _sdpa_masked(q, k, v, row_ptr, col_idx, bq, bk):
    """Library routine: torch SDPA (fp64, CPU) with the block mask expanded to tokens."""
    B, H, N, d = q.shape
    nqb, nkb = -(-N // bq), -(-N // bk)
    mask = np.zeros((B, H, N, N), dtype=bool)
    for bh in range(B * H):
        b, h = divmod(bh, H)
        for i in range(nqb):
            r = bh * nqb + i
            for j in col_idx[row_ptr[r]:row_ptr[r + 1]]:
                mask[b, h, i * bq:(i + 1) * bq, j * bk:(j + 1) * bk] = True
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=torch.from_numpy(mask)).numpy()


def test_sparse_equals_masked_sdpa():
    w = workloads.small_case(H=2, N=1000, d=32, block_q=64, block_k=32, seed=8,
                             alpha=("uniform", 1.0, 3.0), dtype="f32", grid=(10, 10, 10))
    q, k, v = workloads.make_qkv(w)
    r = oracle.route(q, k, w.block_q, w.block_k, 0.8)
    assert r["nnz"] < w.rows * w.nkb       # genuinely sparse
    o = oracle.sparse_attention(q, k, v, r["row_ptr"], r["col_idx"], w.block_q, w.block_k)
    ref = _sdpa_masked(q, k, v, r["row_ptr"], r["col_idx"], w.block_q, w.block_k)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_dense_gate_full_coverage():
    g = GOLD["dense_gate"]
    torch.manual_seed(0)
    q, k, v = (torch.randn(g["B"], g["H"], g["L"], g["D"]) for _ in range(3))
    dense = torch.nn.functional.scaled_dot_product_attention(q.double(), k.double(), v.double()).numpy()
    r = oracle.route(q.numpy(), k.numpy(), g["block"], g["block"], 1.0)
    o = oracle.sparse_attention(q.numpy(), k.numpy(), v.numpy(), r["row_ptr"], r["col_idx"],
                                g["block"], g["block"])
    assert np.abs(o - dense).max() < g["max_abs"]
    assert np.abs(o - dense).max() < 1e-12   # fp64 on both sides
    np.testing.assert_allclose(oracle.dense_attention(q.numpy(), k.numpy(), v.numpy()), dense,
                               rtol=0, atol=1e-12)


def test_zero_keys_average_kept_values():
    rng = np.random.default_rng(9)
    N, d, bq, bk = 300, 16, 64, 32        # 10 key blocks, last one 12 tokens
    q = rng.standard_normal((1, 1, N, d))
    k = np.zeros((1, 1, N, d))
    v = rng.standard_normal((1, 1, N, d))
    # every score is 0, every block has equal importance (uniform): p=0.35 keeps blocks 0..3
    r = oracle.route(q, k, bq, bk, 0.35)
    assert all(row.tolist() == [0, 1, 2, 3] for row in r["kept"][0])
    o = oracle.sparse_attention(q, k, v, r["row_ptr"], r["col_idx"], bq, bk)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0, :128].mean(0), (N, d)), atol=1e-14)
    # p = 1: mean over all N real tokens, including the 12-token tail block
    r1 = oracle.route(q, k, bq, bk, 1.0)
    o1 = oracle.sparse_attention(q, k, v, r1["row_ptr"], r1["col_idx"], bq, bk)
    np.testing.assert_allclose(o1[0, 0], np.broadcast_to(v[0, 0].mean(0), (N, d)), atol=1e-14)


def test_single_token_block_returns_its_value():
    rng = np.random.default_rng(10)
    N, d = 65, 8                          # two key blocks of 64; block 1 holds one token
    q = np.zeros((1, 1, N, d)); q[..., 0] = 1.0
    k = np.zeros((1, 1, N, d)); k[0, 0, 64, 0] = 400.0
    v = rng.standard_normal((1, 1, N, d))
    r = oracle.route(q, k, 64, 64, 0.5)
    assert all(row.tolist() == [1] for row in r["kept"][0])
    o = oracle.sparse_attention(q, k, v, r["row_ptr"], r["col_idx"], 64, 64)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0, 64], (N, d)), atol=0)
