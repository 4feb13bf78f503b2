"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the same
seeded inputs.  CSR: bit-exact except disagreements where the cumulative mass is within
1e-5 of p (counted) and fp near-ties (reported); attention: max-abs <= 2e-2 and
mean-abs <= 2e-3 for bf16 inputs, max-abs <= 1e-4 for fp32 inputs, measured with the
oracle's CSR fed to the GPU so routing and attention are checked independently."""
import math
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import workloads
from _parity import (BF16_MAX_ABS, BF16_MEAN_ABS, F32_MAX_ABS, bf16_half_ulp, classify_rows, merge, record)

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import top_block_sparse_pooled_amd as fv

DEV = torch.device("cuda:0")


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t.float()
    return t.to(DEV).contiguous()


def gpu_route(qd, kd, w, p):
    """GPU routing through the C ABI; also asserts that the routing left no internal-error status."""
    ws = torch.empty(fv.route_ws_bytes(1, w.H, w.N, w.d, w.block_q, w.block_k), dtype=torch.uint8, device=DEV)
    csr = fv.route(qd, kd, w.block_q, w.block_k, p, ws=ws)
    assert fv.ws_status(ws, "route") == 0
    rp = csr.row_ptr.cpu().numpy().astype(np.int64)
    ci = csr.col_idx[: int(rp[-1])].cpu().numpy().astype(np.int64)
    hl = csr.head_load.cpu().numpy().astype(np.int64)
    return csr, rp, ci, hl


def check_csr_invariants(rp, ci, hl, w):
    nqb, nkb = w.nqb, w.nkb
    assert rp[0] == 0 and np.all(np.diff(rp) >= 1)
    assert ci.size == rp[-1]
    assert ci.min() >= 0 and ci.max() < nkb
    for r in range(rp.size - 1):
        seg = ci[rp[r]:rp[r + 1]]
        if seg.size > 1:
            assert np.all(np.diff(seg) > 0), f"row {r} not ascending"
    per_head = np.add.reduceat(np.diff(rp), np.arange(0, rp.size - 1, nqb))
    np.testing.assert_array_equal(hl, per_head)
    assert hl.sum() == rp[-1]


SMALL = [
    # (label, workload factory, p)
    ("tiny_f32_p0.9", lambda: workloads.get("tiny_f32_n1024"), 0.9),
    ("tiny_f32_p1.0", lambda: workloads.get("tiny_f32_n1024"), 1.0),
    ("bf16_h3_n3000_d128", lambda: workloads.small_case(3, 3000, 128, 64, 64, 21, ("uniform", 0.0, 4.0),
                                                        "bf16", (3, 20, 50)), 0.9),
    ("bf16_h2_n5000_bq128", lambda: workloads.small_case(2, 5000, 128, 128, 64, 22, ("loguniform", 0.1, 6.0),
                                                         "bf16", (5, 20, 50)), 0.95),
    ("bf16_h2_n2000_d64_bk32", lambda: workloads.small_case(2, 2000, 64, 64, 32, 23, ("uniform", 0.0, 3.0),
                                                            "bf16", (5, 20, 20)), 0.9),
    ("bf16_h2_n1500_bq32_bk32", lambda: workloads.small_case(2, 1500, 128, 32, 32, 24, ("uniform", 0.5, 3.0),
                                                             "bf16", (3, 10, 50)), 0.8),
    ("f32_h2_n700_d128_bq128", lambda: workloads.small_case(2, 700, 128, 128, 64, 25, ("uniform", 0.0, 3.0),
                                                            "f32", (7, 10, 10)), 0.9),
    ("bf16_h2_n40_short", lambda: workloads.small_case(2, 40, 128, 64, 64, 26, ("uniform", 0.0, 3.0),
                                                       "bf16", (1, 5, 8)), 0.5),
    ("bf16_h2_n2100_d64", lambda: workloads.small_case(2, 2100, 64, 64, 64, 28, ("uniform", 0.0, 3.0),
                                                       "bf16", (5, 20, 21)), 0.9),
    ("bf16_h2_n1800_bq32", lambda: workloads.small_case(2, 1800, 128, 32, 64, 29, ("uniform", 0.5, 3.0),
                                                        "bf16", (3, 20, 30)), 0.85),
    ("bf16_h2_n3000_p1e-6", lambda: workloads.small_case(2, 3000, 128, 64, 64, 32, ("uniform", 0.0, 3.0),
                                                         "bf16", (3, 20, 50)), 1e-6),
    ("bf16_h2_n3000_p0.999999", lambda: workloads.small_case(2, 3000, 128, 64, 64, 33, ("uniform", 0.0, 3.0),
                                                             "bf16", (3, 20, 50)), 0.999999),
    ("bf16_h1_n32760_bk32_nkb1024", lambda: workloads.small_case(1, 32760, 128, 64, 32, 30, ("uniform", 0.0, 4.0),
                                                                 "bf16", (21, 30, 52)), 0.9),
    ("bf16_h2_n22050_bk32_nkb690", lambda: workloads.small_case(2, 22050, 128, 64, 32, 31, ("uniform", 0.0, 3.0),
                                                                "bf16", (21, 30, 35)), 0.85),
    ("bf16_h1_n75600_nkb1182", lambda: workloads.small_case(1, 75600, 128, 64, 64, 27, ("uniform", 0.0, 3.0),
                                                            "bf16", (21, 45, 80)), 0.9),
    # rows of 2,400 key blocks: the longest rows resolved wholly in registers
    ("bf16_h1_n76800_bk32_nkb2400", lambda: workloads.small_case(1, 76800, 128, 64, 32, 40, ("uniform", 0.0, 3.0),
                                                                 "bf16", (20, 48, 80)), 0.9),
    # more heads (B*H = 8, 16, 24)
    ("bf16_h8_n3000", lambda: workloads.small_case(8, 3000, 128, 64, 64, 35, ("uniform", 0.0, 4.0),
                                                         "bf16", (3, 20, 50)), 0.9),
    ("bf16_h16_n1500_d64_bk32", lambda: workloads.small_case(16, 1500, 64, 64, 32, 36, ("uniform", 0.5, 3.0),
                                                                   "bf16", (3, 10, 50)), 0.85),
    ("f32_h8_n700_bq128", lambda: workloads.small_case(8, 700, 128, 128, 64, 37, ("uniform", 0.0, 3.0),
                                                             "f32", (7, 10, 10)), 0.9),
    ("bf16_h8_n22050_bk32_nkb690", lambda: workloads.small_case(8, 22050, 128, 64, 32, 38, ("uniform", 0.0, 3.0),
                                                                      "bf16", (21, 30, 35)), 0.85),
    ("bf16_h24_n4000_bq128", lambda: workloads.small_case(24, 4000, 128, 128, 64, 39, ("loguniform", 0.1, 6.0),
                                                                "bf16", (4, 20, 50)), 0.95),
]


@pytest.mark.parametrize("label,make,p", SMALL, ids=[c[0] for c in SMALL])
def test_route_parity_small(label, make, p):
    w = make()
    say(f"route {label} H={w.H} N={w.N} d={w.d} bq={w.block_q} bk={w.block_k} p={p}")
    q, k = workloads.make_qkv(w, which=(0, 1))
    csr, rp, ci, hl = gpu_route(to_dev(q, w.dtype), to_dev(k, w.dtype), w, p)
    check_csr_invariants(rp, ci, hl, w)
    res = dict(exact=0, excused_A=0, neartie_B=0, fail=0, fail_rows=[])
    for h in range(w.H):
        _, diag = oracle.route_head(q[0, h], k[0, h], w.block_q, w.block_k, p, diagnostics=True)
        res = merge(res, classify_rows(rp, ci, diag, p, row_offset=h * w.nqb))
    record(f"route/{label}", dict(rows=w.rows, kept_frac=float(rp[-1]) / (w.rows * w.nkb), **res))
    assert res["fail"] == 0, res["fail_rows"]
    if p >= 1.0:
        assert rp[-1] == w.rows * w.nkb


def test_pool_parity():
    for w in (workloads.small_case(2, 3000, 128, 64, 64, 31, ("uniform", 0.0, 3.0), "bf16", (3, 20, 50)),
              workloads.small_case(2, 1000, 64, 32, 32, 32, ("uniform", 0.0, 3.0), "f32", (10, 10, 10))):
        for blk in (w.block_q, 128):
            say(f"pool {w.name} block={blk}")
            (x,) = workloads.make_qkv(w, which=(0,))
            got = fv.pool(to_dev(x, w.dtype), blk).cpu().numpy()
            for h in range(w.H):
                ref = oracle.pool_blocks(x[0, h], blk)
                np.testing.assert_allclose(got[0, h], ref, rtol=1e-15, atol=1e-15)


def _golden_case_tensors(kind):
    """The closed-form constructions of tests/golden/closed_forms.json at supported sizes."""
    d = 64
    if kind == "uniform":
        N = 1024
        rng = np.random.default_rng(2)
        q = rng.standard_normal((1, 1, N, d)).astype(np.float32)
        k = np.zeros((1, 1, N, d), np.float32)
        return q, k, 64, 64
    if kind == "tie":
        N = 128
        q = np.zeros((1, 1, N, d), np.float32); q[..., 0] = 1.0
        k = np.zeros((1, 1, N, d), np.float32)
        k[0, 0, 32:64, 0] = 8 * math.log(4.0)     # score = 1 * 8 ln4 / sqrt(64) = ln 4
        k[0, 0, 96:128, 0] = 8 * math.log(4.0)
        return q, k, 128, 32
    if kind == "logistic":
        N = 64
        q = np.zeros((1, 1, N, d), np.float32); q[..., 0] = 1.0
        k = np.zeros((1, 1, N, d), np.float32)
        k[0, 0, :32, 0] = 8 * math.log(9.0)       # masses 0.9 / 0.1
        return q, k, 64, 32
    raise ValueError(kind)


GOLD_CASES = [("uniform", 0.9, 15, list(range(15))), ("uniform", 0.5, 8, list(range(8))),
              ("uniform", 0.0625, 1, [0]), ("uniform", 0.0626, 2, [0, 1]), ("uniform", 1.0, 16, list(range(16))),
              ("tie", 0.3, 1, [1]), ("tie", 0.7, 2, [1, 3]), ("tie", 0.85, 3, [0, 1, 3]),
              ("logistic", 0.85, 1, [0]), ("logistic", 0.95, 2, [0, 1])]


@pytest.mark.parametrize("kind,p,count,kept", GOLD_CASES, ids=[f"{c[0]}_p{c[1]}" for c in GOLD_CASES])
def test_route_closed_forms_exact(kind, p, count, kept):
    say(f"closed form {kind} p={p}")
    q, k, bq, bk = _golden_case_tensors(kind)
    csr = fv.route(to_dev(q, "f32"), to_dev(k, "f32"), bq, bk, p)
    torch.cuda.synchronize()
    rp = csr.row_ptr.cpu().numpy()
    ci = csr.col_idx.cpu().numpy()
    for r in range(rp.size - 1):
        assert ci[rp[r]:rp[r + 1]].tolist() == kept, (r, ci[rp[r]:rp[r + 1]].tolist())


ATTN_CASES = [c for c in SMALL if not c[0].startswith("bf16_h1_n75600")]


@pytest.mark.parametrize("label,make,p", ATTN_CASES, ids=[c[0] for c in ATTN_CASES])
def test_attention_parity_small(label, make, p):
    w = make()
    say(f"attn {label} H={w.H} N={w.N} d={w.d} bq={w.block_q} bk={w.block_k} p={p}")
    q, k, v = workloads.make_qkv(w)
    r = oracle.route(q, k, w.block_q, w.block_k, p)
    ref = oracle.sparse_attention(q, k, v, r["row_ptr"], r["col_idx"], w.block_q, w.block_k)
    qd, kd, vd = to_dev(q, w.dtype), to_dev(k, w.dtype), to_dev(v, w.dtype)
    csr = fv.Csr.from_host(r["row_ptr"], r["col_idx"], r["head_load"], w.H, w.N, w.block_q, w.block_k, DEV)
    o_t = fv.sparse_attn(qd, kd, vd, csr, out_dtype=torch.float32)
    o = o_t.cpu().numpy()
    if w.dtype == "bf16":
        # the bf16 output is the round-to-nearest-even of the float32 result, bit for bit
        o_b = fv.sparse_attn(qd, kd, vd, csr)
        assert o_b.dtype == torch.bfloat16 and torch.equal(o_b, o_t.to(torch.bfloat16))
    err = np.abs(o - ref)
    record(f"attn/{label}", dict(max_abs=float(err.max()), mean_abs=float(err.mean()), nnz=int(r["nnz"])))
    if w.dtype == "bf16":
        assert err.max() <= BF16_MAX_ABS and err.mean() <= BF16_MEAN_ABS
    else:
        assert err.max() <= F32_MAX_ABS
    # end to end: GPU routing feeding GPU attention
    csr_g = fv.route(qd, kd, w.block_q, w.block_k, p)
    o2 = fv.sparse_attn(qd, kd, vd, csr_g, out_dtype=torch.float32).cpu().numpy()
    rp = csr_g.row_ptr.cpu().numpy()
    same = np.array_equal(rp, r["row_ptr"]) and np.array_equal(csr_g.col_idx[: rp[-1]].cpu().numpy(), r["col_idx"])
    if same:
        e2 = np.abs(o2 - ref)
        assert e2.max() <= (BF16_MAX_ABS if w.dtype == "bf16" else F32_MAX_ABS)


def test_p1_equals_dense_fp32():
    """The tutorial's full-coverage gate on the GPU: every block kept == dense attention."""
    torch.manual_seed(0)
    say("dense gate B=2 H=4 L=512 D=64 fp32")
    q, k, v = (torch.randn(2, 4, 512, 64) for _ in range(3))
    dense = torch.nn.functional.scaled_dot_product_attention(q.double(), k.double(), v.double()).numpy()
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    csr = fv.route(qd, kd, 64, 64, 1.0)
    assert csr.nnz() == 2 * 4 * 8 * 8
    o = fv.sparse_attn(qd, kd, vd, csr).cpu().numpy()
    assert np.abs(o - dense).max() < 1e-4


def test_worklist_exact_and_schedules():
    """Every work-list order, at row level and at the unit sizes the attention kernels consume,
    bit-exact against the oracle's orders; the per-XCD queue starts of RLB as well."""
    w = workloads.small_case(12, 6000, 128, 64, 64, 41, ("loguniform", 0.1, 6.0), "bf16", (6, 20, 50))
    say(f"worklist {w.name}")
    q, k = workloads.make_qkv(w, which=(0, 1))
    csr, rp, ci, hl = gpu_route(to_dev(q, w.dtype), to_dev(k, w.dtype), w, 0.9)
    for G in (1, 2, 4):
        ngroups = -(-w.nqb // G)
        expect = {"lpt": oracle.lpt_units(rp, w.nqb, G), "identity": np.arange(w.H * ngroups),
                  "head_lpt": oracle.head_lpt_units(rp, w.nqb, G), "head_desc": oracle.head_desc_units(rp, w.nqb, G),
                  "xcd": np.arange(w.H * ngroups)}
        for sched, ex in expect.items():
            got = fv.worklist(csr, sched, G).cpu().numpy().astype(np.int64)
            np.testing.assert_array_equal(got, ex, err_msg=f"{sched} G={G}")
        wl, ctl = fv.worklist(csr, "rlb", G, with_control=True)
        ex, starts = oracle.rlb_units(rp, w.nqb, G, 8)
        np.testing.assert_array_equal(wl.cpu().numpy().astype(np.int64), ex, err_msg=f"rlb G={G}")
        np.testing.assert_array_equal(ctl[16:25].cpu().numpy().astype(np.int64), starts)
    assert np.array_equal(oracle.lpt_units(rp, w.nqb, 1), oracle.lpt_worklist(rp))
    # the plan of the bf16 attention: units of 128 query rows (G = 128 / block_q = 2 here)
    qd = to_dev(q, w.dtype)
    ws = fv.attn_ws(qd, csr)
    units = w.H * -(-w.nqb // 2)
    for sched, fn in (("lpt", oracle.lpt_units), ("head_lpt", oracle.head_lpt_units)):
        fv.attn_plan(qd, csr, ws, sched)
        got = fv.plan_worklist(csr, ws, units).cpu().numpy().astype(np.int64)
        np.testing.assert_array_equal(got, fn(rp, w.nqb, 2))
    fv.attn_plan(qd, csr, ws, "rlb")
    np.testing.assert_array_equal(fv.plan_worklist(csr, ws, units).cpu().numpy().astype(np.int64),
                                  oracle.rlb_units(rp, w.nqb, 2, 8)[0])


def test_plan_mismatch_is_refused():
    """A plan built for bf16 units and run on float32 inputs of the same shape (and the reverse)
    is refused by the kernels: status bit set, output untouched."""
    w = workloads.small_case(2, 1500, 64, 64, 64, 61, ("uniform", 0.0, 3.0), "bf16", (3, 10, 50))
    say(f"plan mismatch {w.name}")
    q, k, v = workloads.make_qkv(w)
    qb, kb, vb = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    qf, kf, vf = to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32")
    csr = fv.route(qb, kb, 64, 64, 0.9)
    ws = fv.attn_ws(qb, csr)
    fv.attn_plan(vb, csr, ws, "identity")
    assert fv.ws_status(ws, "attn") == 0
    sentinel = torch.full(qf.shape, 7.0, dtype=torch.float32, device=DEV)
    fv.attn_run(qf, kf, vf, csr, ws, out=sentinel)
    assert fv.ws_status(ws, "attn") == fv.STATUS["plan_mismatch"]
    assert bool((sentinel == 7.0).all())
    fv.attn_plan(vf, csr, ws, "identity")
    sent_b = torch.full(qb.shape, 3.0, dtype=torch.bfloat16, device=DEV)
    fv.attn_run(qb, kb, vb, csr, ws, out=sent_b)
    assert fv.ws_status(ws, "attn") == fv.STATUS["plan_mismatch"]
    assert bool((sent_b == 3.0).all())
    # a matching plan runs and clears the status
    fv.attn_plan(vb, csr, ws, "identity")
    o = fv.attn_run(qb, kb, vb, csr, ws)
    assert fv.ws_status(ws, "attn") == 0
    assert torch.equal(o, fv.sparse_attn(qb, kb, vb, csr))


def test_determinism_schedule_independence_and_trace():
    w = workloads.small_case(3, 4000, 128, 64, 64, 51, ("uniform", 0.0, 4.0), "bf16", (4, 20, 50))
    say(f"determinism {w.name}")
    q, k, v = workloads.make_qkv(w)
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    csr = fv.route(qd, kd, 64, 64, 0.9)
    csr2 = fv.route(qd, kd, 64, 64, 0.9)
    assert torch.equal(csr.row_ptr, csr2.row_ptr) and torch.equal(csr.col_idx[: csr.nnz()], csr2.col_idx[: csr.nnz()])
    outs = [fv.sparse_attn(qd, kd, vd, csr, schedule=s)
            for s in ("lpt", "lpt", "identity", "head_lpt", "xcd", "rlb", "head_desc")]
    outs.append(fv.sparse_attn(qd, kd, vd, csr, schedule="lpt", grid=7))
    for o in outs[1:]:
        assert torch.equal(outs[0], o)
    ws = fv.attn_ws(qd, csr)
    fv.attn_plan(vd, csr, ws, "lpt")
    for _ in range(3):   # the plan can be run repeatedly (the kernel resets its tile counter)
        assert torch.equal(fv.attn_run(qd, kd, vd, csr, ws), outs[0])
    units = w.H * -(-w.nqb // 2)            # bf16 work units: pairs of 64-row query blocks
    trace = torch.zeros(w.rows * 4, dtype=torch.int64, device=DEV)
    o_t = fv.sparse_attn(qd, kd, vd, csr, trace=trace)
    assert torch.equal(o_t, outs[0])
    tr = trace.cpu().numpy().reshape(-1, 4).view(np.uint64)
    assert sorted(tr[:units, 3].astype(np.int64).tolist()) == list(range(units))   # every unit exactly once
    assert np.all(tr[:units, 2] >= tr[:units, 1]) and np.all(tr[units:] == 0)
    # per-XCD queues with stealing: every tile exactly once, repeatable on one plan
    for sched in ("xcd", "rlb"):
        fv.attn_plan(vd, csr, ws, sched)
        for _ in range(3):
            trace.zero_()
            assert torch.equal(fv.attn_run(qd, kd, vd, csr, ws, trace=trace), outs[0])
            tr = trace.cpu().numpy().reshape(-1, 4).view(np.uint64)
            assert sorted(tr[:units, 3].astype(np.int64).tolist()) == list(range(units))
        assert fv.ws_status(ws, "attn") == 0
    # a trace smaller than 4 records per unit is refused before any launch
    with pytest.raises(fv.FvAttnError):
        fv.sparse_attn(qd, kd, vd, csr, trace=torch.zeros(4 * units - 1, dtype=torch.int64, device=DEV))


# ------------------------------------------------------------------ full-size workloads
FULL = [("wan1p3b_n32760", 0.9), ("wan14b_n32760", 0.90), ("wan14b_n32760", 0.95), ("wan14b_n32760", 1.0),
        ("wan14b_n32760_bk32", 0.9), ("wan14b_n75600", 0.9), ("wan14b_n75600_bk32", 0.9),
        ("skew_n75600_bq128", 0.95),
        # single heads of 102,400 and 131,040 tokens (1600 and 4095 key blocks)
        ("long_h1_n102400", 0.9), ("long_h1_n131040_bk32", 0.9)]

LONG = {
    "long_h1_n102400": lambda: workloads.small_case(1, 102400, 128, 64, 64, 81, ("uniform", 0.0, 3.0), "bf16",
                                                    (32, 40, 80)),
    "long_h1_n131040_bk32": lambda: workloads.small_case(1, 131040, 128, 64, 32, 82, ("uniform", 0.0, 3.0), "bf16",
                                                         (39, 40, 84)),
}


@pytest.mark.parametrize("name,p", FULL, ids=[f"{n}_p{p}" for n, p in FULL])
def test_full_size(name, p):
    """Full-size workload in the benchmark's launch configuration.  The oracle routes every head,
    and every CSR row is compared; attention is compared on the heaviest row, the lightest row,
    the ragged last query block and one random block of every head, for the float32 output and
    for the bf16 output (which must also be the round-to-nearest-even of the float32 output)."""
    w = LONG[name]() if name in LONG else workloads.get(name)
    say(f"full {name} p={p}: generating inputs")
    q, k, v = workloads.make_qkv(w)
    qd, kd, vd = to_dev(q, w.dtype), to_dev(k, w.dtype), to_dev(v, w.dtype)
    say(f"full {name} p={p}: GPU route + attention")
    csr, rp, ci, hl = gpu_route(qd, kd, w, p)
    check_csr_invariants(rp, ci, hl, w)
    o32 = fv.sparse_attn(qd, kd, vd, csr, out_dtype=torch.float32)
    o16 = fv.sparse_attn(qd, kd, vd, csr)
    assert torch.equal(o16, o32.to(torch.bfloat16)), "bf16 output is not the RNE of the float32 output"
    torch.cuda.synchronize()
    res = dict(exact=0, excused_A=0, neartie_B=0, fail=0, fail_rows=[])
    e32, e16, e16x = [], [], []
    rng = np.random.default_rng(99)
    nrows_att = 0
    for h in range(w.H):
        if h % 10 == 0:
            say(f"full {name} p={p}: oracle heads {h}..{min(h + 9, w.H - 1)}")
        kept, diag = oracle.route_head(q[0, h], k[0, h], w.block_q, w.block_k, p, diagnostics=True)
        res = merge(res, classify_rows(rp, ci, diag, p, row_offset=h * w.nqb))
        counts = diag["counts"]
        rows = {w.nqb - 1, int(np.argmax(counts)), int(np.argmin(counts)), int(rng.integers(0, w.nqb))}
        # the GPU attention ran on the GPU's CSR: compare rows whose kept set agrees
        sel = {i: kept[i] for i in rows
               if np.array_equal(ci[rp[h * w.nqb + i]:rp[h * w.nqb + i + 1]], kept[i])}
        ref = oracle.sparse_attention_rows(q[0, h], k[0, h], v[0, h], w.block_q, w.block_k, sel)
        for i, oi in ref.items():
            s0 = i * w.block_q
            e32.append(np.abs(o32[0, h, s0:s0 + oi.shape[0]].cpu().numpy() - oi).ravel())
            d16 = np.abs(o16[0, h, s0:s0 + oi.shape[0]].float().cpu().numpy() - oi)
            e16.append(d16.ravel())
            e16x.append((d16 - bf16_half_ulp(oi)).ravel())
            nrows_att += 1
    err32, err16, err16x = np.concatenate(e32), np.concatenate(e16), np.concatenate(e16x)
    kept_frac = float(rp[-1]) / (w.rows * w.nkb)
    per_head = (hl / (w.nqb * w.nkb)).tolist()
    record(f"full/{name}/p{p}", dict(rows=w.rows, nnz=int(rp[-1]), kept_frac=kept_frac,
                                     head_kept_min=float(min(per_head)), head_kept_max=float(max(per_head)),
                                     head_load_max_over_mean=float(hl.max() / hl.mean()), attn_rows=nrows_att,
                                     attn_max_abs=float(err32.max()), attn_mean_abs=float(err32.mean()),
                                     bf16_max_abs=float(err16.max()), bf16_mean_abs=float(err16.mean()),
                                     bf16_max_abs_beyond_rounding=float(err16x.max()),
                                     bf16_mean_abs_beyond_rounding=float(np.maximum(err16x, 0.0).mean()), **res))
    assert res["fail"] == 0, res["fail_rows"]
    assert res["exact"] + res["excused_A"] + res["neartie_B"] == w.rows
    assert err32.max() <= BF16_MAX_ABS and err32.mean() <= BF16_MEAN_ABS
    # bf16 output: both bounds on the error beyond the half ulp that rounding the exact result to
    # bf16 itself leaves (one bf16 ulp is 2^-6 for |o| in [2, 4) and 2^-4 in [8, 16), so the raw
    # bf16 error of any correct output can exceed the stated bounds); the raw figures are recorded
    assert err16x.max() <= BF16_MAX_ABS
    assert np.maximum(err16x, 0.0).mean() <= BF16_MEAN_ABS
