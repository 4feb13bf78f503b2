"""GPU parity of SASA (fvattn_route_sasa) against the fp64 oracle's route_sasa: augmented
CSR, per-head loads and per-group budgets.  Selection across rows compares importances that
the two sides compute with different rounding (the GPU's softmax denominator is an exact
fixed-point sum, the oracle's a float64 sum), so a candidate whose importance lies within
1e-12 (relative) of its group's threshold may fall on either side; such rows are counted as
near-ties and everything else must match exactly."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import workloads
from _parity import record

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import top_block_sparse_pooled_amd as fv

DEV = torch.device("cuda:0")
NEAR = 1e-12


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t.float()
    return t.to(DEV).contiguous()


def gpu_sasa(qd, kd, bq, bk, p, groups, alpha, tau, critical=0, **variant):
    added = torch.zeros(groups, dtype=torch.int32, device=DEV)
    B, H, N, d = qd.shape
    ws = torch.empty(fv.lib().fvattn_route_sasa_ws_bytes(B, H, N, d, bq, bk, groups), dtype=torch.uint8, device=DEV)
    csr = fv.route_sasa(qd, kd, bq, bk, p, groups=groups, alpha=alpha, tau=tau, critical=critical, added=added,
                        ws=ws, **variant)
    assert fv.ws_status(ws, "route") == 0
    rp = csr.row_ptr.cpu().numpy().astype(np.int64)
    ci = csr.col_idx[: int(rp[-1])].cpu().numpy().astype(np.int64)
    hl = csr.head_load.cpu().numpy().astype(np.int64)
    return rp, ci, hl, added.cpu().numpy().astype(np.int64)


def compare(rp, ci, ref, nqb, groups, H):
    """Rows that differ from the oracle; each must differ only in candidates at their group's
    threshold importance (near-ties).  Returns (exact rows, near-tie rows, failing rows)."""
    base = ref["base_kept"]
    P = ref["P"]
    thr = {}
    for g in range(groups):
        added = []
        for h in range(H):
            if h * groups // H != g:
                continue
            for i in range(nqb):
                extra = np.setdiff1d(ref["kept"][h][i], base[h][i])
                added += list(P[h][i, extra])
        thr[g] = min(added) if added else None
    exact = near = 0
    fail = []
    for h in range(H):
        g = h * groups // H
        for i in range(nqb):
            r = h * nqb + i
            got = ci[rp[r]:rp[r + 1]]
            want = ref["kept"][h][i]
            if np.array_equal(got, want):
                exact += 1
                continue
            diff = np.setxor1d(got, want)
            t = thr[g]
            if t is not None and np.all(np.abs(P[h][i, diff] - t) <= NEAR * t):
                near += 1
            else:
                fail.append(r)
    return exact, near, fail


def _two_heads_case():
    nb, b, d = 16, 32, 64
    N = nb * b
    q = np.ones((1, 2, N, d), np.float32)
    k = np.zeros((1, 2, N, d), np.float32)
    k[0, 0, 7 * b:8 * b] = 3.0
    return q, k, b


def test_sasa_closed_form_on_gpu():
    """Head 0 keeps one block per row, head 1 eight; with two groups, alpha = 0.5, head 0 gains
    56 blocks taken from its tied candidates in row order (rows 0-2 whole, 11 in row 3)."""
    q, k, b = _two_heads_case()
    rp, ci, hl, added = gpu_sasa(to_dev(q, "f32"), to_dev(k, "f32"), b, b, 0.5, 2, 0.5, 0.0)
    assert added.tolist() == [56, 0] and hl.tolist() == [72, 128]
    for i in range(3):
        assert list(ci[rp[i]:rp[i + 1]]) == list(range(16))
    assert list(ci[rp[3]:rp[4]]) == list(range(12))
    for i in range(4, 16):
        assert list(ci[rp[i]:rp[i + 1]]) == [7]
    rp, ci, hl, added = gpu_sasa(to_dev(q, "f32"), to_dev(k, "f32"), b, b, 0.5, 2, 1.0, 0.0, critical=160)
    assert added.tolist() == [144, 32] and hl.tolist() == [160, 160]
    rp, ci, hl, added = gpu_sasa(to_dev(q, "f32"), to_dev(k, "f32"), b, b, 0.5, 2, 0.5, 0.9)
    assert added.tolist() == [0, 0] and hl.tolist() == [16, 128]


CASES = [
    ("bf16_h4_n3000", lambda: workloads.small_case(4, 3000, 128, 64, 64, 51, ("uniform", 0.0, 4.0), "bf16",
                                                   (3, 20, 50)), 0.9),
    ("bf16_h6_n2000_bq128", lambda: workloads.small_case(6, 2000, 128, 128, 64, 52, ("loguniform", 0.1, 6.0),
                                                         "bf16", (5, 20, 20)), 0.9),
    ("f32_h4_n1000_d64", lambda: workloads.small_case(4, 1000, 64, 32, 32, 53, ("uniform", 0.0, 3.0), "f32",
                                                      (4, 10, 25)), 0.8),
    ("bf16_h2_n22050_bk32_nkb690", lambda: workloads.small_case(2, 22050, 128, 64, 32, 54, ("uniform", 0.0, 3.5),
                                                                "bf16", (21, 30, 35)), 0.85),
    ("bf16_h2_n69120_bq128_bk32_nkb2160", lambda: workloads.small_case(2, 69120, 128, 128, 32, 55,
                                                                       ("uniform", 0.5, 3.0), "bf16",
                                                                       (24, 36, 80)), 0.9),
    ("bf16_h2_n83200_bq128_bk32_nkb2600", lambda: workloads.small_case(2, 83200, 128, 128, 32, 56,
                                                                       ("uniform", 0.5, 3.0), "bf16",
                                                                       (20, 52, 80)), 0.9),
]
SETTINGS = [
    ("g2_a0.5", dict(groups=2, alpha=0.5, tau=0.0), {}),
    ("g4_a1_t0.1", dict(groups=4, alpha=1.0, tau=0.1), {}),
    ("g2_a0.3_topk8_w1", dict(groups=2, alpha=0.3, tau=0.0), dict(mode="topk", topk=8, window=1)),
]


@pytest.mark.parametrize("slabel,sopts,variant", SETTINGS, ids=[x[0] for x in SETTINGS])
@pytest.mark.parametrize("label,make,p", CASES, ids=[c[0] for c in CASES])
def test_sasa_parity_small(label, make, p, slabel, sopts, variant):
    w = make()
    groups = min(sopts["groups"], w.H)
    say(f"sasa {label} {slabel} H={w.H} N={w.N} bq={w.block_q} bk={w.block_k} p={p}")
    q, k = workloads.make_qkv(w, which=(0, 1))
    rp, ci, hl, added = gpu_sasa(to_dev(q, w.dtype), to_dev(k, w.dtype), w.block_q, w.block_k, p, groups,
                                 sopts["alpha"], sopts["tau"], **variant)
    ref = oracle.route_sasa(q, k, w.block_q, w.block_k, p, groups, sopts["alpha"], sopts["tau"], **variant)
    assert added.tolist() == ref["budgets"]
    exact, near, fail = compare(rp, ci, ref, w.nqb, groups, w.H)
    record(f"sasa/{label}/{slabel}", dict(rows=w.rows, added=int(added.sum()), exact=exact, near_tie=near,
                                          fail=len(fail)))
    assert not fail, f"rows differ beyond near-ties: {fail[:10]}"
    if near == 0:
        np.testing.assert_array_equal(hl, ref["head_load"])
    # loads of every group stay within the critical path
    for g in range(groups):
        assert sum(hl[h] for h in range(w.H) if h * groups // w.H == g) <= ref["critical"]


def test_sasa_full_size_one_group():
    """The benchmark layer (H=40, N=32760, p=0.9) in 8 groups, alpha 0.5, trigger 0.05: every
    row of one group (heads 15-19) against the oracle, and the budgets of all groups."""
    w = workloads.get("wan14b_n32760")
    groups, alpha, tau = 8, 0.5, 0.05
    say(f"sasa full {w.name} groups={groups}")
    q, k = workloads.make_qkv(w, which=(0, 1))
    rp, ci, hl, added = gpu_sasa(to_dev(q, "bf16"), to_dev(k, "bf16"), w.block_q, w.block_k, 0.9, groups, alpha, tau)
    # per-head Top-p loads from the oracle for the budgets
    kept, P = [], []
    for h in range(w.H):
        kh, extra = oracle.route_head(q[0, h], k[0, h], w.block_q, w.block_k, 0.9, diagnostics=(15 <= h < 20))
        kept.append(kh)
        P.append(extra["P"] if extra is not None else None)
    loads = [sum(len(x) for x in kh) for kh in kept]
    L = [sum(loads[h] for h in range(w.H) if h * groups // w.H == g) for g in range(groups)]
    crit = max(L)
    want = [oracle.sasa_budget(crit - L[g], crit, alpha, tau) for g in range(groups)]
    assert added.tolist() == want
    sub, bud, _ = oracle.sasa_augment([kept[h] for h in range(15, 20)], [P[h] for h in range(15, 20)], 1, alpha,
                                      tau, critical=crit)
    assert bud == [want[3]]
    ref = dict(kept=sub, base_kept=[kept[h] for h in range(15, 20)], P=[P[h] for h in range(15, 20)])
    rows = slice(15 * w.nqb, 20 * w.nqb + 1)
    rp5 = rp[rows] - rp[15 * w.nqb]
    ci5 = ci[rp[15 * w.nqb]:rp[20 * w.nqb]]
    exact, near, fail = compare(rp5, ci5, ref, w.nqb, 1, 5)
    record(f"sasa/full/{w.name}/g8_a0.5_t0.05", dict(added=[int(x) for x in added], rows_checked=5 * w.nqb,
                                                     exact=exact, near_tie=near, fail=len(fail)))
    assert not fail
