"""Plain, slow, fp64 CPU oracle of the Top-p block-sparse attention hot path.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the CPU
baseline of the benchmark; never by the GPU library.  It shares no code with
the HIP kernels.  Every function works on numpy arrays in float64 and follows
the pages step by step, using numpy primitives (mean, matmul, exp, a stable
argsort, cumsum) and no blocking, fusion or reordering of its own.

Sources (titles of the web pages the method is taken from):
  [FVAttn]  "腾讯+中山大学新作：视频生成提速2.11×，靠的是RLB和SASA" (PaperDaily summary
            of FVAttn, arXiv:2607.16190), section "AI视频生成的阿喀琉斯之踵", the
            paragraph describing Top-p routing; and the RLB section (per-head load).
  [TUTOR]   the engineering tutorial page on accelerating video generation, section
            5.2 "块稀疏注意力的教学实现" (block mean-pooling, 1/sqrt(d) block scores)
            and section 5.3 "正确性验证" (full coverage must equal dense attention).

Readings of points the pages leave open (each also listed in the design notes):
  * importance of key block j for query block i = softmax over j of the scaled
    pooled score  qbar_i . kbar_j / sqrt(d)  (pooled form of [TUTOR] 5.2, with the
    softmax that turns scores into a mass summing to 1, as [FVAttn] accumulates
    "importance" up to p);
  * pooling is the mean over the block's REAL tokens (the ragged last block is
    divided by its own length; padding never enters);
  * "reaches p" means cumulative mass >= p; the kept set is the shortest prefix
    of the descending order that reaches p; ties in importance go to the lower
    block index; p >= 1 keeps every block, and if rounding leaves the total below
    p every block is kept;
  * routing is per (head, query block): all tokens of a query block share the
    kept set;
  * attention is exact, non-causal softmax attention with scale 1/sqrt(d) over
    the real tokens of the kept key blocks.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence

import numpy as np


# --------------------------------------------------------------------------
# Step 1: fixed-size blocks ([FVAttn] Top-p paragraph: keys/values are cut into
# fixed blocks of e.g. 32 or 64 tokens).
# --------------------------------------------------------------------------
def block_bounds(n_tokens: int, block: int) -> List[tuple]:
    """[(start, end)] of the consecutive blocks of `block` tokens; the last may be short."""
    nb = -(-n_tokens // block)
    return [(i * block, min((i + 1) * block, n_tokens)) for i in range(nb)]


# --------------------------------------------------------------------------
# Step 2: block mean-pooling ([TUTOR] 5.2: each block is summarised by the mean
# vector of its tokens, which keeps the scoring cheap).
# --------------------------------------------------------------------------
def pool_blocks(x: np.ndarray, block: int) -> np.ndarray:
    """x [N, d] -> [nb, d]: mean over the real tokens of each block."""
    x = np.asarray(x, dtype=np.float64)
    return np.stack([x[s:e].mean(axis=0) for s, e in block_bounds(x.shape[0], block)])


# --------------------------------------------------------------------------
# Step 3: scaled block scores ([TUTOR] 5.2: pooled-q . pooled-k divided by sqrt(d)).
# --------------------------------------------------------------------------
def block_scores(qbar: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    d = qbar.shape[1]
    return (qbar @ kbar.T) / math.sqrt(d)


# --------------------------------------------------------------------------
# Step 4: importance = softmax over key blocks (max subtracted), rows sum to 1.
# --------------------------------------------------------------------------
def block_importance(scores: np.ndarray) -> np.ndarray:
    m = scores.max(axis=-1, keepdims=True)
    e = np.exp(scores - m)
    return e / e.sum(axis=-1, keepdims=True)


# --------------------------------------------------------------------------
# Step 5: descending order of importance, ties to the lower block index
# ([FVAttn]: blocks are ranked by importance in descending order).  A stable
# sort on -P keeps equal keys in ascending index order.
# --------------------------------------------------------------------------
def routing_order(P: np.ndarray) -> np.ndarray:
    return np.argsort(-P, axis=-1, kind="stable")


# --------------------------------------------------------------------------
# Step 6: the Top-p cut ([FVAttn]: blocks are taken in that order until the
# cumulative importance reaches p; the kept set is the smallest such set).
# --------------------------------------------------------------------------
def topp_count(P_sorted_row: np.ndarray, p: float) -> int:
    """k* = smallest k >= 1 with sum of the first k sorted masses >= p.
    p >= 1, or a total that rounding leaves below p, keeps every block."""
    n = P_sorted_row.shape[0]
    if p >= 1.0:
        return n
    S = np.cumsum(P_sorted_row)          # S[k-1] = mass of the first k blocks
    hit = np.nonzero(S >= p)[0]
    return int(hit[0]) + 1 if hit.size else n


# --------------------------------------------------------------------------
# Routing variants (the hot path's next rows).  [FVAttn] contrasts Top-p with a
# fixed Top-k; [TUTOR] 5.2 keeps the top-k key blocks by pooled score and adds
# a local window of neighbouring blocks as a floor.  Readings:
#   * mode "topk": the first min(k, nkb) blocks of the descending order (the
#     same order and tie rule as Top-p; softmax is monotone, so this is the
#     top-k by pooled score);
#   * a clamp k_min <= k* <= k_max on the Top-p count (k_max = 0: none), taken
#     as the first k* blocks of the order;
#   * window w > 0: key blocks within w blocks of those that overlap the query
#     block's token span are always kept (union with the selection); w = 0 adds
#     nothing.  With equal block sizes this is [TUTOR]'s i-w .. i+w.
# --------------------------------------------------------------------------
def selection_count(P_sorted_row: np.ndarray, mode: str = "topp", p: float = 0.9,
                    topk: int = 0, k_min: int = 1, k_max: int = 0) -> int:
    """Number of leading blocks of the descending order the selection keeps."""
    n = P_sorted_row.shape[0]
    if mode == "topk":
        return min(int(topk), n)
    c = topp_count(P_sorted_row, p)
    c = max(c, int(k_min))
    if k_max > 0:
        c = min(c, int(k_max))
    return min(c, n)


def window_blocks(i: int, n_tokens: int, block_q: int, block_k: int, window: int) -> np.ndarray:
    """Key blocks forced by a local window of `window` blocks around query block i."""
    if window <= 0:
        return np.zeros(0, dtype=np.int64)
    nkb = -(-n_tokens // block_k)
    s0, e0 = i * block_q, min((i + 1) * block_q, n_tokens)
    jlo, jhi = s0 // block_k, (e0 - 1) // block_k      # key blocks overlapping the span
    return np.arange(max(0, jlo - window), min(nkb - 1, jhi + window) + 1, dtype=np.int64)


def route_head(q_h: np.ndarray, k_h: np.ndarray, block_q: int, block_k: int, p: float,
               diagnostics: bool = False, mode: str = "topp", topk: int = 0, k_min: int = 1,
               k_max: int = 0, window: int = 0):
    """Routing of one head: q_h, k_h [N, d].  Returns (kept, extra) where kept is a
    list over query blocks of ascending int arrays of kept key-block indices.
    With diagnostics, extra = dict(order, cum, counts, P).  mode / topk / k_min /
    k_max / window select a routing variant (defaults: plain Top-p)."""
    qbar = pool_blocks(q_h, block_q)
    kbar = pool_blocks(k_h, block_k)
    P = block_importance(block_scores(qbar, kbar))
    order = routing_order(P)
    N = q_h.shape[0]
    kept, counts, cums = [], [], []
    for i in range(P.shape[0]):
        Ps = P[i, order[i]]
        c = selection_count(Ps, mode, p, topk, k_min, k_max)
        sel = order[i, :c]
        win = window_blocks(i, N, block_q, block_k, window)
        kept.append(np.union1d(sel, win).astype(np.int64))
        counts.append(c)
        if diagnostics:
            cums.append(np.cumsum(Ps))
    extra = None
    if diagnostics:
        extra = dict(order=order, cum=np.array(cums), counts=np.array(counts), P=P,
                     qbar=qbar, kbar=kbar)
    return kept, extra


def csr_rows(kept_per_head: Sequence[Sequence[np.ndarray]]):
    """Build the CSR of key-block indices over rows r = head * nqb + i, plus the
    per-head load ([FVAttn] RLB section: a head's load is the number of blocks it
    must compute, read off its sparse mask)."""
    counts = [len(k) for head in kept_per_head for k in head]
    row_ptr = np.zeros(len(counts) + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(counts)
    col_idx = (np.concatenate([k for head in kept_per_head for k in head]).astype(np.int64)
               if counts and row_ptr[-1] > 0 else np.zeros(0, dtype=np.int64))
    head_load = np.array([sum(len(k) for k in head) for head in kept_per_head], dtype=np.int64)
    return row_ptr, col_idx, head_load


def route(q: np.ndarray, k: np.ndarray, block_q: int, block_k: int, p: float,
          diagnostics: bool = False, **variant):
    """q, k [B, H, N, d] -> dict(row_ptr, col_idx, head_load, nnz[, per-head diagnostics]).
    `variant` (mode, topk, k_min, k_max, window) selects a routing variant."""
    B, H, N, d = q.shape
    kept_all, diags = [], []
    for b in range(B):
        for h in range(H):
            kept, extra = route_head(q[b, h], k[b, h], block_q, block_k, p, diagnostics, **variant)
            kept_all.append(kept)
            diags.append(extra)
    row_ptr, col_idx, head_load = csr_rows(kept_all)
    out = dict(row_ptr=row_ptr, col_idx=col_idx, head_load=head_load, nnz=int(row_ptr[-1]),
               kept=kept_all)
    if diagnostics:
        out["diag"] = diags
    return out


# --------------------------------------------------------------------------
# Step 8: exact softmax attention over the kept blocks ([FVAttn]: attention then
# runs only over the selected blocks; the sparse computation itself is exact).
# Two-pass softmax (max, then exp and sum), scale 1/sqrt(d), fp64.
# --------------------------------------------------------------------------
def _attend(q_rows: np.ndarray, keys: np.ndarray, vals: np.ndarray) -> np.ndarray:
    d = q_rows.shape[1]
    s = (q_rows @ keys.T) / math.sqrt(d)
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    return (w @ vals) / w.sum(axis=1, keepdims=True)


def sparse_attention_rows(q_h, k_h, v_h, block_q: int, block_k: int,
                          kept_rows: dict) -> dict:
    """For one head: {query block i: o [len(block i), d]} for the rows in kept_rows
    (i -> ascending kept key-block indices)."""
    q_h = np.asarray(q_h, dtype=np.float64)
    k_h = np.asarray(k_h, dtype=np.float64)
    v_h = np.asarray(v_h, dtype=np.float64)
    N = q_h.shape[0]
    qb = block_bounds(N, block_q)
    kb = block_bounds(N, block_k)
    out = {}
    for i, kept in kept_rows.items():
        s0, e0 = qb[i]
        tok = np.concatenate([np.arange(*kb[j]) for j in kept])
        out[i] = _attend(q_h[s0:e0], k_h[tok], v_h[tok])
    return out


def sparse_attention(q, k, v, row_ptr, col_idx, block_q: int, block_k: int) -> np.ndarray:
    """Full output o [B, H, N, d] (fp64) of block-sparse attention given a CSR over
    rows r = (b*H + h) * nqb + i."""
    B, H, N, d = q.shape
    nqb = -(-N // block_q)
    o = np.zeros((B, H, N, d), dtype=np.float64)
    qb = block_bounds(N, block_q)
    for b in range(B):
        for h in range(H):
            r0 = (b * H + h) * nqb
            rows = {i: np.asarray(col_idx[row_ptr[r0 + i]:row_ptr[r0 + i + 1]]) for i in range(nqb)}
            res = sparse_attention_rows(q[b, h], k[b, h], v[b, h], block_q, block_k, rows)
            for i, oi in res.items():
                o[b, h, qb[i][0]:qb[i][1]] = oi
    return o


def dense_attention(q, k, v) -> np.ndarray:
    """Textbook softmax(q k^T / sqrt(d)) v per (b, h), fp64."""
    B, H, N, d = q.shape
    o = np.zeros((B, H, N, d), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            o[b, h] = _attend(np.asarray(q[b, h], np.float64), np.asarray(k[b, h], np.float64),
                              np.asarray(v[b, h], np.float64))
    return o


# --------------------------------------------------------------------------
# Step 7: one-GPU analogue of the runtime load balancing ([FVAttn] RLB section:
# the heaviest work is moved first).  Tiles (rows) ordered by kept-block count,
# longest first; equal counts keep ascending row id.
# --------------------------------------------------------------------------
def lpt_worklist(row_ptr: np.ndarray) -> np.ndarray:
    counts = np.diff(np.asarray(row_ptr, dtype=np.int64))
    return np.argsort(-counts, kind="stable").astype(np.int64)


# --------------------------------------------------------------------------
# Work units of the attention and their orders ([FVAttn] RLB section: a
# head's load is the number of blocks it must compute; the balancer moves the
# heaviest heads first, each to the least loaded rank).  A unit is G adjacent
# query blocks of one head (G = 1: one CSR row); unit u = head * ngroups + g
# holds query blocks g*G .. min(g*G + G, nqb) - 1 of its head, and its work is
# the number of kept (query block, key block) pairs of those rows.
# --------------------------------------------------------------------------
def unit_work(row_ptr: np.ndarray, nqb: int, G: int) -> np.ndarray:
    counts = np.diff(np.asarray(row_ptr, dtype=np.int64))
    nh = counts.size // nqb
    ngroups = -(-nqb // G)
    work = np.zeros(nh * ngroups, dtype=np.int64)
    for h in range(nh):
        for g in range(ngroups):
            work[h * ngroups + g] = counts[h * nqb + g * G: h * nqb + min(g * G + G, nqb)].sum()
    return work


def head_loads(row_ptr: np.ndarray, nqb: int) -> np.ndarray:
    counts = np.diff(np.asarray(row_ptr, dtype=np.int64))
    return counts.reshape(-1, nqb).sum(axis=1)


def lpt_units(row_ptr: np.ndarray, nqb: int, G: int) -> np.ndarray:
    """Units by work, heaviest first; equal work keeps ascending unit id."""
    return np.argsort(-unit_work(row_ptr, nqb, G), kind="stable").astype(np.int64)


def heads_by_load(row_ptr: np.ndarray, nqb: int) -> np.ndarray:
    """Heads by load, heaviest first; equal loads keep ascending head id."""
    return np.argsort(-head_loads(row_ptr, nqb), kind="stable").astype(np.int64)


def head_lpt_units(row_ptr: np.ndarray, nqb: int, G: int) -> np.ndarray:
    """Heads heaviest first; within a head its units heaviest first (ties by id)."""
    work = unit_work(row_ptr, nqb, G)
    ngroups = -(-nqb // G)
    out = []
    for h in heads_by_load(row_ptr, nqb):
        us = np.arange(h * ngroups, (h + 1) * ngroups)
        out.extend(us[np.argsort(-work[us], kind="stable")].tolist())
    return np.array(out, dtype=np.int64)


def head_desc_units(row_ptr: np.ndarray, nqb: int, G: int) -> np.ndarray:
    """Heads heaviest first; a head's units in id order."""
    ngroups = -(-nqb // G)
    return np.array([h * ngroups + g for h in heads_by_load(row_ptr, nqb) for g in range(ngroups)],
                    dtype=np.int64)


def rlb_assign(loads: np.ndarray, n_bins: int):
    """Greedy of the RLB section on one machine: heads taken heaviest first (ties:
    lower id), each given to the bin (rank) with the least load so far (ties: lower
    bin).  Returns (bin of each head, list per bin of its heads in assignment order)."""
    loads = np.asarray(loads, dtype=np.int64)
    bin_load = [0] * n_bins
    bins = [[] for _ in range(n_bins)]
    where = np.zeros(loads.size, dtype=np.int64)
    for h in np.argsort(-loads, kind="stable"):
        b = min(range(n_bins), key=lambda x: (bin_load[x], x))
        bins[b].append(int(h))
        bin_load[b] += int(loads[h])
        where[h] = b
    return where, bins


def rlb_units(row_ptr: np.ndarray, nqb: int, G: int, n_bins: int = 8):
    """Per-XCD queues: heads assigned by rlb_assign over the n_bins XCDs, each queue
    its heads in assignment order with a head's units in id order, queues
    concatenated.  Returns (work list, start of each queue + [total])."""
    ngroups = -(-nqb // G)
    _, bins = rlb_assign(head_loads(row_ptr, nqb), n_bins)
    order, starts = [], []
    for b in bins:
        starts.append(len(order))
        for h in b:
            order.extend(range(h * ngroups, (h + 1) * ngroups))
    starts.append(len(order))
    return np.array(order, dtype=np.int64), np.array(starts, dtype=np.int64)


# --------------------------------------------------------------------------
# SASA, slack-aware sparsity augmentation ([FVAttn] SASA section).  After load
# balancing every rank knows its own block count and the largest one (the
# critical path); the difference is its slack.  A rank adds the highest-
# importance blocks that Top-p left out, taken from the candidate lists of all
# its heads in the routing's importance order, as many as its slack allows,
# scaled by an augmentation coefficient, and only when the slack passes a
# trigger threshold.  Readings for one GPU:
#   * ranks are R contiguous groups of the layer's heads (the per-rank share of
#     sequence parallelism); the critical path is the largest group load, or a
#     caller-given value (e.g. gathered from the other ranks);
#   * load = kept (query block, key block) pairs; slack = critical - load;
#     budget = floor(alpha * slack) if slack >= tau * critical and slack > 0,
#     else 0;
#   * candidates = every unselected (row, key block) of the group's rows,
#     ranked by importance P descending, ties to the lower row, then the lower
#     key block; the first `budget` are added.
# --------------------------------------------------------------------------
def sasa_budget(slack: int, critical: int, alpha: float, tau: float) -> int:
    """Blocks a group may add: floor(alpha * slack) when the slack passes the trigger."""
    if slack <= 0 or slack < tau * critical:
        return 0
    return int(math.floor(alpha * slack))


def sasa_augment(kept_per_head, P_per_head, groups: int, alpha: float, tau: float,
                 critical: int = 0):
    """kept_per_head[h][i]: ascending kept key blocks; P_per_head[h]: importance
    [nqb, nkb].  Returns (augmented kept lists, per-group blocks added, critical path)."""
    H = len(kept_per_head)
    nqb, nkb = P_per_head[0].shape
    group_of = [h * groups // H for h in range(H)]
    loads = [sum(len(x) for x in kept_per_head[h]) for h in range(H)]
    L = [sum(loads[h] for h in range(H) if group_of[h] == g) for g in range(groups)]
    crit = int(critical) if critical > 0 else max(L)
    out = [[np.asarray(x, dtype=np.int64) for x in head] for head in kept_per_head]
    budgets = []
    for g in range(groups):
        slack = crit - L[g]
        budget = sasa_budget(slack, crit, alpha, tau)
        if budget <= 0:
            budgets.append(0)
            continue
        cands = []
        for h in range(H):
            if group_of[h] != g:
                continue
            for i in range(nqb):
                keep = np.zeros(nkb, dtype=bool)
                keep[kept_per_head[h][i]] = True
                for j in np.nonzero(~keep)[0]:
                    cands.append((-P_per_head[h][i, j], h * nqb + i, int(j)))
        cands.sort()
        budget = min(budget, len(cands))      # a group cannot add more blocks than it left out
        budgets.append(budget)
        for _, row, j in cands[:budget]:
            h, i = divmod(row, nqb)
            out[h][i] = np.union1d(out[h][i], [j]).astype(np.int64)
    return out, budgets, crit


def route_sasa(q, k, block_q: int, block_k: int, p: float, groups: int, alpha: float, tau: float,
               critical: int = 0, **variant):
    """Routing (Top-p or a variant) followed by SASA over the heads of B x H."""
    B, H, N, d = q.shape
    kept_all, P_all = [], []
    for b in range(B):
        for h in range(H):
            kept, extra = route_head(q[b, h], k[b, h], block_q, block_k, p, True, **variant)
            kept_all.append(kept)
            P_all.append(extra["P"])
    aug, budgets, crit = sasa_augment(kept_all, P_all, groups, alpha, tau, critical)
    row_ptr, col_idx, head_load = csr_rows(aug)
    return dict(row_ptr=row_ptr, col_idx=col_idx, head_load=head_load, nnz=int(row_ptr[-1]),
                kept=aug, base_kept=kept_all, P=P_all, budgets=budgets, critical=crit)
