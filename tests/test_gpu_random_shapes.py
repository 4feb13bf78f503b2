"""GPU parity over seeded random shapes: head dim, block sizes, token grid (ragged tails, a
sequence shorter than one block), p, dtype and the spread of the per-head position weight are
drawn from a fixed generator.  Each case checks the routing CSR against the oracle (bit-exact
rows, with the excused and near-tie classes of the other parity tests) and the attention on
the oracle's CSR against the oracle's attention, to the same tolerances."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import workloads
from _parity import BF16_MAX_ABS, BF16_MEAN_ABS, F32_MAX_ABS, classify_rows, merge, record

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


def _draw_cases(n=16, seed=20261203):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        bq = int(rng.choice([32, 64, 128]))
        bk = int(rng.choice([32, 64]))
        T, Y, X = int(rng.integers(1, 6)), int(rng.integers(1, 18)), int(rng.integers(1, 26))
        if i == 0:
            T, Y, X = 1, 1, 23          # shorter than any block
        if i >= 10:
            T, Y, X = T + 2, Y + 15, X + 20   # larger grids: many tiles per unit, ragged tails
        N = T * Y * X
        H = int(rng.integers(1, 4))
        p = 1.0 if i == 1 else round(float(rng.uniform(0.5, 0.99)), 3)
        dtype = "f32" if i in (2, 7) else "bf16"
        hi = round(float(rng.uniform(0.5, 5.0)), 2)
        alpha = ("loguniform", 0.1, hi + 0.1) if i % 3 == 0 else ("uniform", 0.0, hi)
        label = f"r{i}_{dtype}_h{H}_n{N}_d{d}_bq{bq}_bk{bk}_p{p}"
        cases.append((label, (H, N, d, bq, bk, 900 + i, alpha, dtype, (T, Y, X)), p))
    return cases


CASES = _draw_cases()


@pytest.mark.parametrize("label,args,p", CASES, ids=[c[0] for c in CASES])
def test_random_shape_parity(label, args, p):
    w = workloads.small_case(*args)
    say(f"random {label}")
    q, k, v = workloads.make_qkv(w)
    qd, kd, vd = to_dev(q, w.dtype), to_dev(k, w.dtype), to_dev(v, w.dtype)
    # routing
    ws = torch.empty(fv.route_ws_bytes(1, w.H, w.N, w.d, w.block_q, w.block_k), dtype=torch.uint8, device=DEV)
    csr_g = fv.route(qd, kd, w.block_q, w.block_k, p, ws=ws)
    assert fv.ws_status(ws, "route") == 0
    rp = csr_g.row_ptr.cpu().numpy().astype(np.int64)
    ci = csr_g.col_idx[: int(rp[-1])].cpu().numpy().astype(np.int64)
    hl = csr_g.head_load.cpu().numpy().astype(np.int64)
    assert rp[0] == 0 and np.all(np.diff(rp) >= 1) and hl.sum() == rp[-1]
    res = dict(exact=0, excused_A=0, neartie_B=0, fail=0, fail_rows=[])
    for h in range(w.H):
        _, diag = oracle.route_head(q[0, h], k[0, h], w.block_q, w.block_k, p, diagnostics=True)
        res = merge(res, classify_rows(rp, ci, diag, p, row_offset=h * w.nqb))
    # attention on the oracle's CSR
    r = oracle.route(q, k, w.block_q, w.block_k, p)
    ref = oracle.sparse_attention(q, k, v, r["row_ptr"], r["col_idx"], w.block_q, w.block_k)
    csr = fv.Csr.from_host(r["row_ptr"], r["col_idx"], r["head_load"], w.H, w.N, w.block_q, w.block_k, DEV)
    o = fv.sparse_attn(qd, kd, vd, csr, out_dtype=torch.float32).cpu().numpy()
    err = np.abs(o - ref)
    record(f"random/{label}", dict(rows=w.rows, max_abs=float(err.max()), mean_abs=float(err.mean()), **res))
    assert res["fail"] == 0, res["fail_rows"]
    if res["excused_A"] == 0 and res["neartie_B"] == 0:
        np.testing.assert_array_equal(hl, r["head_load"])
    if w.dtype == "bf16":
        assert err.max() <= BF16_MAX_ABS and err.mean() <= BF16_MEAN_ABS
    else:
        assert err.max() <= F32_MAX_ABS


def test_batch_equals_heads():
    """B > 1 is more heads: the same 4 heads routed and attended as [2, 2, N, d] and as
    [1, 4, N, d] give identical CSRs, loads and outputs, and the CSR matches the oracle."""
    w = workloads.small_case(4, 1700, 128, 64, 64, 950, ("uniform", 0.0, 3.5), "bf16", (2, 25, 34))
    say("batch B=2 H=2 vs B=1 H=4, N=1700")
    q, k, v = workloads.make_qkv(w)
    outs = []
    for shape in ((1, 4), (2, 2)):
        qd, kd, vd = (to_dev(x.reshape(*shape, w.N, w.d), "bf16") for x in (q, k, v))
        csr = fv.route(qd, kd, w.block_q, w.block_k, 0.85)
        o = fv.sparse_attn(qd, kd, vd, csr)
        torch.cuda.synchronize()
        rp = csr.row_ptr.cpu().numpy()
        outs.append((rp, csr.col_idx[: int(rp[-1])].cpu().numpy(), csr.head_load.cpu().numpy(),
                     o.reshape(1, 4, w.N, w.d).cpu()))
    (rp1, ci1, hl1, o1), (rp2, ci2, hl2, o2) = outs
    np.testing.assert_array_equal(rp1, rp2)
    np.testing.assert_array_equal(ci1, ci2)
    np.testing.assert_array_equal(hl1, hl2)
    assert torch.equal(o1, o2)
    r = oracle.route(q, k, w.block_q, w.block_k, 0.85)
    np.testing.assert_array_equal(rp1.astype(np.int64), r["row_ptr"])
    np.testing.assert_array_equal(ci1.astype(np.int64), r["col_idx"])
