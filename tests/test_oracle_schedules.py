"""Pins of the oracle's work-unit orders (the one-GPU analogue of the FVAttn summary's runtime
load balancing, section 'RLB': per-head load = blocks to compute; heaviest heads first, each to the
least loaded rank).  Hand-derived cases in tests/golden/schedules.json, invariants that define the
orders, the list-scheduling bound of the greedy, and planted mistakes that a pin must catch."""
import json
import os

import numpy as np
import pytest

import oracle
import oracle.topp_oracle as T

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "schedules.json")))


def _row_ptr(counts):
    return np.concatenate([[0], np.cumsum(np.asarray(counts, dtype=np.int64))])


def test_rlb_assign_hand_example():
    g = GOLD["rlb_assign_3_bins"]
    where, bins = oracle.rlb_assign(np.array(g["loads"]), 3)
    assert bins == g["bins"]
    loads = np.array(g["loads"])
    assert [int(loads[b].sum()) for b in bins] == g["bin_loads"]
    for b, hs in enumerate(bins):
        assert all(where[h] == b for h in hs)


def test_unit_work_and_orders_hand_example():
    g = GOLD["unit_work"]
    rp = _row_ptr(g["counts"])
    assert oracle.unit_work(rp, g["nqb"], g["G"]).tolist() == g["work"]
    assert oracle.lpt_units(rp, g["nqb"], g["G"]).tolist() == g["lpt"]
    assert oracle.head_lpt_units(rp, g["nqb"], g["G"]).tolist() == g["head_lpt"]
    assert oracle.head_desc_units(rp, g["nqb"], g["G"]).tolist() == g["head_desc"]


def _random_csr(seed, nh=13, nqb=37):
    rng = np.random.default_rng(seed)
    # heads of very different density, as the skewed workloads have
    dens = rng.uniform(0.02, 1.0, size=nh)
    counts = np.concatenate([rng.binomial(60, d, size=nqb) + 1 for d in dens])
    return _row_ptr(counts), nqb, counts


@pytest.mark.parametrize("G", [1, 2, 4])
def test_unit_orders_invariants(G):
    rp, nqb, counts = _random_csr(3 + G)
    nh = counts.size // nqb
    ngroups = -(-nqb // G)
    work = oracle.unit_work(rp, nqb, G)
    assert work.sum() == rp[-1] and work.size == nh * ngroups
    lpt = oracle.lpt_units(rp, nqb, G)
    assert sorted(lpt.tolist()) == list(range(work.size))
    wv = work[lpt]
    assert np.all(np.diff(wv) <= 0)
    assert all(a < b for a, b in zip(lpt[:-1], lpt[1:]) if work[a] == work[b])
    if G == 1:   # rows: the row-level LPT order
        assert lpt.tolist() == oracle.lpt_worklist(rp).tolist()
    hl = oracle.head_loads(rp, nqb)
    for order in (oracle.head_lpt_units(rp, nqb, G), oracle.head_desc_units(rp, nqb, G)):
        assert sorted(order.tolist()) == list(range(work.size))
        heads = order // ngroups
        # heads appear as contiguous runs, heaviest first, ties by id
        runs = [int(h) for i, h in enumerate(heads) if i == 0 or heads[i - 1] != h]
        assert len(runs) == nh and np.all(np.diff(hl[runs]) <= 0)
        assert all(a < b for a, b in zip(runs[:-1], runs[1:]) if hl[a] == hl[b])
    hlpt = oracle.head_lpt_units(rp, nqb, G)
    for h in range(nh):
        seg = hlpt[hlpt // ngroups == h]
        assert np.all(np.diff(work[seg]) <= 0)
    hd = oracle.head_desc_units(rp, nqb, G)
    for h in range(nh):
        assert np.all(np.diff(hd[hd // ngroups == h]) == 1)


@pytest.mark.parametrize("nbins", [3, 8])
def test_rlb_units_invariants_and_greedy_bound(nbins):
    rp, nqb, counts = _random_csr(11, nh=40, nqb=20)
    G = 2
    ngroups = -(-nqb // G)
    wl, starts = oracle.rlb_units(rp, nqb, G, nbins)
    assert sorted(wl.tolist()) == list(range(40 * ngroups))
    assert starts[0] == 0 and starts[-1] == wl.size and np.all(np.diff(starts) >= 0)
    hl = oracle.head_loads(rp, nqb)
    bin_loads = []
    for b in range(nbins):
        q = wl[starts[b]:starts[b + 1]]
        heads = q // ngroups
        # whole heads, each head's units in id order
        runs = [int(h) for i, h in enumerate(heads) if i == 0 or heads[i - 1] != h]
        for h in runs:
            seg = q[heads == h]
            assert seg.tolist() == list(range(h * ngroups, (h + 1) * ngroups))
        # heads of a queue in assignment order: heaviest first
        assert np.all(np.diff(hl[runs]) <= 0)
        bin_loads.append(int(hl[runs].sum()))
    # list scheduling bound of the greedy: max bin load <= mean + largest head load
    assert max(bin_loads) <= sum(bin_loads) / nbins + hl.max()
    # heaviest first: the nbins heaviest heads open the nbins queues (ties by id)
    first = sorted(int(wl[starts[b]]) // ngroups for b in range(nbins))
    assert first == sorted(oracle.heads_by_load(rp, nqb)[:nbins].tolist())


def _mutant_fails(monkeypatch, name, fn):
    monkeypatch.setattr(T, name, fn)
    monkeypatch.setattr(oracle, name, fn)
    failed = False
    for test in (test_rlb_assign_hand_example, test_unit_work_and_orders_hand_example,
                 lambda: test_unit_orders_invariants(2), lambda: test_rlb_units_invariants_and_greedy_bound(3)):
        try:
            test()
        except AssertionError:
            failed = True
    monkeypatch.undo()
    return failed


def test_planted_schedule_mistakes_are_caught(monkeypatch):
    orig_assign = T.rlb_assign

    def assign_most_loaded(loads, n_bins):          # sends each head to the MOST loaded bin
        loads = np.asarray(loads, dtype=np.int64)
        bl, bins, where = [0] * n_bins, [[] for _ in range(n_bins)], np.zeros(loads.size, np.int64)
        for h in np.argsort(-loads, kind="stable"):
            b = max(range(n_bins), key=lambda x: (bl[x], -x))
            bins[b].append(int(h)); bl[b] += int(loads[h]); where[h] = b
        return where, bins

    def assign_lightest_first(loads, n_bins):       # takes heads lightest first
        loads = np.asarray(loads, dtype=np.int64)
        bl, bins, where = [0] * n_bins, [[] for _ in range(n_bins)], np.zeros(loads.size, np.int64)
        for h in np.argsort(loads, kind="stable"):
            b = min(range(n_bins), key=lambda x: (bl[x], x))
            bins[b].append(int(h)); bl[b] += int(loads[h]); where[h] = b
        return where, bins

    def assign_ties_high(loads, n_bins):            # ties to the higher bin
        loads = np.asarray(loads, dtype=np.int64)
        bl, bins, where = [0] * n_bins, [[] for _ in range(n_bins)], np.zeros(loads.size, np.int64)
        for h in np.argsort(-loads, kind="stable"):
            b = min(range(n_bins), key=lambda x: (bl[x], -x))
            bins[b].append(int(h)); bl[b] += int(loads[h]); where[h] = b
        return where, bins

    def work_off_by_one(row_ptr, nqb, G):            # unit spans G + 1 rows
        counts = np.diff(np.asarray(row_ptr, dtype=np.int64))
        nh, ngroups = counts.size // nqb, -(-nqb // G)
        return np.array([counts[h * nqb + g * G: h * nqb + min(g * G + G + 1, nqb)].sum()
                         for h in range(nh) for g in range(ngroups)], dtype=np.int64)

    def lpt_ties_high(row_ptr, nqb, G):              # equal work: higher id first
        w = T.unit_work(row_ptr, nqb, G)
        return np.array(sorted(range(w.size), key=lambda u: (-w[u], -u)), dtype=np.int64)

    def heads_ascending(row_ptr, nqb):               # lightest head first
        return np.argsort(T.head_loads(row_ptr, nqb), kind="stable").astype(np.int64)

    assert _mutant_fails(monkeypatch, "rlb_assign", assign_most_loaded)
    assert _mutant_fails(monkeypatch, "rlb_assign", assign_lightest_first)
    assert _mutant_fails(monkeypatch, "rlb_assign", assign_ties_high)
    assert _mutant_fails(monkeypatch, "unit_work", work_off_by_one)
    assert _mutant_fails(monkeypatch, "lpt_units", lpt_ties_high)
    assert _mutant_fails(monkeypatch, "heads_by_load", heads_ascending)
    assert T.rlb_assign is orig_assign
