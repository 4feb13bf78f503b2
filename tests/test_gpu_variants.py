"""GPU parity of the routing variants (fixed top-k, clamped Top-p count, local window) through
fvattn_route_ex, against the fp64 oracle run with the same variant: CSR and per-head loads
bit-exact."""
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


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t.float()
    return t.to(DEV).contiguous()


def gpu_route(qd, kd, bq, bk, p, **variant):
    B, H, N, d = qd.shape
    ws = torch.empty(fv.route_ws_bytes(B, H, N, d, bq, bk), dtype=torch.uint8, device=DEV)
    csr = fv.route(qd, kd, bq, bk, p, ws=ws, **variant)
    assert fv.ws_status(ws, "route") == 0
    rp = csr.row_ptr.cpu().numpy().astype(np.int64)
    ci = csr.col_idx[: int(rp[-1])].cpu().numpy().astype(np.int64)
    hl = csr.head_load.cpu().numpy().astype(np.int64)
    return rp, ci, hl


CASES = [
    ("bf16_h3_n3000_d128", lambda: workloads.small_case(3, 3000, 128, 64, 64, 41, ("uniform", 0.0, 4.0),
                                                        "bf16", (3, 20, 50))),
    ("bf16_h2_n5000_bq128", lambda: workloads.small_case(2, 5000, 128, 128, 64, 42, ("loguniform", 0.1, 6.0),
                                                         "bf16", (5, 20, 50))),
    ("bf16_h2_n1500_bq32_bk32", lambda: workloads.small_case(2, 1500, 64, 32, 32, 43, ("uniform", 0.5, 3.0),
                                                             "bf16", (3, 10, 50))),
    ("f32_h2_n1000_d64", lambda: workloads.small_case(2, 1000, 64, 64, 64, 44, ("uniform", 0.0, 3.0),
                                                      "f32", (4, 10, 25))),
    ("bf16_h1_n22050_bk32_nkb690", lambda: workloads.small_case(1, 22050, 128, 64, 32, 46, ("uniform", 0.0, 3.0),
                                                                "bf16", (21, 30, 35))),
    ("bf16_h1_n75600_nkb1182", lambda: workloads.small_case(1, 75600, 128, 64, 64, 45, ("uniform", 0.0, 3.0),
                                                            "bf16", (21, 45, 80))),
    ("bf16_h1_n69120_bk32_nkb2160", lambda: workloads.small_case(1, 69120, 128, 64, 32, 47, ("uniform", 0.0, 3.0),
                                                                 "bf16", (24, 36, 80))),
    ("bf16_h1_n76800_bk32_nkb2400", lambda: workloads.small_case(1, 76800, 128, 64, 32, 48, ("uniform", 0.0, 3.0),
                                                                 "bf16", (20, 48, 80))),
    # rows of 2,600 key blocks: part in registers, part in the scratch
    ("bf16_h1_n83200_bq128_bk32_nkb2600", lambda: workloads.small_case(1, 83200, 128, 128, 32, 49,
                                                                       ("uniform", 0.0, 3.0), "bf16",
                                                                       (20, 52, 80))),
]

VARIANTS = [
    ("topk1", 0.9, dict(mode="topk", topk=1)),
    ("topk7", 0.9, dict(mode="topk", topk=7)),
    ("topk_all", 0.9, dict(mode="topk", topk=5000)),
    ("clamp3_10", 0.9, dict(k_min=3, k_max=10)),
    ("clamp_min12", 0.6, dict(k_min=12)),
    ("p1_kmax4", 1.0, dict(k_max=4)),
    ("window2", 0.5, dict(window=2)),
    ("topk5_window1", 0.9, dict(mode="topk", topk=5, window=1)),
]


@pytest.mark.parametrize("vlabel,p,variant", VARIANTS, ids=[v[0] for v in VARIANTS])
@pytest.mark.parametrize("label,make", CASES, ids=[c[0] for c in CASES])
def test_variant_parity_small(label, make, vlabel, p, variant):
    w = make()
    say(f"route_ex {label} {vlabel} H={w.H} N={w.N} bq={w.block_q} bk={w.block_k} p={p} {variant}")
    q, k = workloads.make_qkv(w, which=(0, 1))
    rp, ci, hl = gpu_route(to_dev(q, w.dtype), to_dev(k, w.dtype), w.block_q, w.block_k, p, **variant)
    ref = oracle.route(q, k, w.block_q, w.block_k, p, **variant)
    bad = [r for r in range(w.rows)
           if not np.array_equal(ci[rp[r]:rp[r + 1]], ref["col_idx"][ref["row_ptr"][r]:ref["row_ptr"][r + 1]])]
    record(f"variant/{label}/{vlabel}", dict(rows=w.rows, nnz=int(rp[-1]), mismatched_rows=len(bad)))
    assert not bad, f"rows differ: {bad[:10]}"
    np.testing.assert_array_equal(rp, ref["row_ptr"])
    np.testing.assert_array_equal(hl, ref["head_load"])


def test_variant_closed_forms_on_gpu():
    """k == 0: every importance ties, so top-k keeps blocks 0..k-1; a window adds i-w .. i+w."""
    N, d, b = 1024, 64, 64
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    k = np.zeros((1, 1, N, d), np.float32)
    qd, kd = to_dev(q, "f32"), to_dev(k, "f32")
    rp, ci, _ = gpu_route(qd, kd, b, b, 0.9, mode="topk", topk=5)
    for r in range(16):
        assert list(ci[rp[r]:rp[r + 1]]) == [0, 1, 2, 3, 4]
    rp, ci, _ = gpu_route(qd, kd, b, b, 0.5, window=2)
    for i in range(16):
        expect = sorted(set(range(8)) | set(range(max(0, i - 2), min(15, i + 2) + 1)))
        assert list(ci[rp[i]:rp[i + 1]]) == expect
    rp, ci, _ = gpu_route(qd, kd, b, b, 0.5, k_max=3)
    for r in range(16):
        assert list(ci[rp[r]:rp[r + 1]]) == [0, 1, 2]


def test_variant_full_size_sampled():
    """The benchmark layer (H=40, N=32760) with top-64 plus a window of 1: CSR rows of three
    sampled heads against the oracle."""
    w = workloads.get("wan14b_n32760")
    variant = dict(mode="topk", topk=64, window=1)
    say(f"route_ex full {w.name} {variant}")
    q, k = workloads.make_qkv(w, which=(0, 1))
    rp, ci, hl = gpu_route(to_dev(q, "bf16"), to_dev(k, "bf16"), w.block_q, w.block_k, 0.9, **variant)
    assert rp[-1] == hl.sum()
    bad = 0
    for h in (3, 19, 33):
        kept, _ = oracle.route_head(q[0, h], k[0, h], w.block_q, w.block_k, 0.9, **variant)
        for i, ks in enumerate(kept):
            r = h * w.nqb + i
            bad += not np.array_equal(ci[rp[r]:rp[r + 1]], ks)
        assert hl[h] == sum(len(x) for x in kept)
    record(f"variant/full/{w.name}/topk64_window1", dict(rows_checked=3 * w.nqb, mismatched_rows=bad))
    assert bad == 0
