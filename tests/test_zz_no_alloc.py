"""The no-allocation attention entry point (fvattn_sparse_attn_noalloc, for callers that cannot
allocate: graph capture, serving loops) against the workspace entry point it varies
(fvattn_sparse_attn), through the C ABI: bitwise-equal outputs on two calls in a row, the
second smaller, for several schedules, both output types and float32 inputs; and against the
oracle within the attention tolerance."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import workloads
from _parity import BF16_MAX_ABS, BF16_MEAN_ABS, F32_MAX_ABS

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


CASES = [   # the second call of each pair is smaller than the first
    (workloads.small_case(4, 6000, 128, 64, 64, 71, ("loguniform", 0.1, 6.0), "bf16", (6, 20, 50)), 0.9),
    (workloads.small_case(2, 1500, 64, 32, 32, 72, ("uniform", 0.5, 3.0), "bf16", (3, 10, 50)), 0.85),
    (workloads.small_case(2, 2100, 128, 128, 64, 73, ("uniform", 0.0, 3.0), "f32", (3, 10, 70)), 0.9),
    (workloads.small_case(1, 700, 64, 64, 64, 74, ("uniform", 0.0, 3.0), "f32", (7, 10, 10)), 0.9),
]


def _run_pair(big, small):
    outs = []
    for w, p in (big, small):
        say(f"noalloc {w.name} p={p}")
        q, k, v = workloads.make_qkv(w)
        qd, kd, vd = to_dev(q, w.dtype), to_dev(k, w.dtype), to_dev(v, w.dtype)
        r = oracle.route(q, k, w.block_q, w.block_k, p)
        csr = fv.Csr.from_host(r["row_ptr"], r["col_idx"], r["head_load"], w.H, w.N, w.block_q, w.block_k, DEV)
        scheds = ("identity", "rlb", "lpt") if w.dtype == "bf16" else ("identity", "lpt")
        for sched in scheds:
            ref = fv.sparse_attn(qd, kd, vd, csr, schedule=sched)
            got = fv.sparse_attn_noalloc(qd, kd, vd, csr, schedule=sched)
            torch.cuda.synchronize()
            assert torch.equal(got, ref), (w.name, sched)
        if w.dtype == "bf16":
            ref32 = fv.sparse_attn(qd, kd, vd, csr, out_dtype=torch.float32)
            got32 = fv.sparse_attn_noalloc(qd, kd, vd, csr, out_dtype=torch.float32)
            assert torch.equal(got32, ref32)
            err = np.abs(got32.cpu().numpy() - oracle.sparse_attention(q, k, v, r["row_ptr"], r["col_idx"],
                                                                       w.block_q, w.block_k))
            assert err.max() <= BF16_MAX_ABS and err.mean() <= BF16_MEAN_ABS
        else:
            err = np.abs(got.cpu().numpy() - oracle.sparse_attention(q, k, v, r["row_ptr"], r["col_idx"],
                                                                     w.block_q, w.block_k))
            assert err.max() <= F32_MAX_ABS
        outs.append(got)
    return outs


def test_noalloc_equals_workspace_entry_point_bf16():
    _run_pair(CASES[0], CASES[1])


def test_noalloc_equals_workspace_entry_point_f32():
    _run_pair(CASES[2], CASES[3])


def test_noalloc_repeated_calls_keep_results():
    """The shared scratch keeps the last call's plan: a call after a larger one, and the larger one
    again, give the same outputs as the first time."""
    first = _run_pair(CASES[0], CASES[1])
    again = _run_pair(CASES[0], CASES[1])
    for a, b in zip(first, again):
        assert torch.equal(a, b)


def test_noalloc_refuses_oversized():
    B, H, N = 1, 300, 81920   # 300 x 1280 rows > FVATTN_NOALLOC_MAX_ROWS; fails validation, nothing launched
    x = torch.zeros(B, H, 64, 64, dtype=torch.bfloat16, device=DEV)   # never read
    csr = fv.Csr(x.new_zeros(1, dtype=torch.int32), x.new_zeros(1, dtype=torch.int32),
                 x.new_zeros(1, dtype=torch.int32), B * H, N, 64, 64, N // 64, N // 64)
    c = csr.c()
    o = fv._OptsC(1, 0, None, 0, -1, 0)
    rc = fv.lib().fvattn_sparse_attn_noalloc(x.data_ptr(), x.data_ptr(), x.data_ptr(), x.data_ptr(), B, H, N, 64, 0,
                                             __import__("ctypes").byref(c), __import__("ctypes").byref(o), None)
    assert rc == -8
