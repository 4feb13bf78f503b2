"""Comparison helpers for the GPU parity tests (inputs/expectations from the oracle only)."""
from __future__ import annotations

import json
import os

import numpy as np

CUT_TOL = 1e-5      # a disagreement is excused only where the cumulative mass lies within 1e-5 of p
TIE_REL = 1e-6      # near-tie between a kept and a dropped block (reported separately)

BF16_MAX_ABS, BF16_MEAN_ABS = 2e-2, 2e-3
F32_MAX_ABS = 1e-4


def bf16_half_ulp(x):
    """Half a unit in the last place of bfloat16 (8 significant bits) at |x|: the error that
    rounding the exact value itself to bf16 may leave (2^(e-8) for |x| in [2^e, 2^(e+1)))."""
    ax = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), np.finfo(np.float32).tiny)
    return np.ldexp(1.0, np.floor(np.log2(ax)).astype(np.int64) - 8)


def classify_rows(gpu_row_ptr, gpu_col_idx, diag, p, row_offset=0):
    """Compare GPU CSR rows of one head with the oracle's routing diagnostics of that head.
    Returns dict(exact, excused_A, neartie_B, fail, fail_rows)."""
    res = dict(exact=0, excused_A=0, neartie_B=0, fail=0, fail_rows=[])
    order, cum, counts, P = diag["order"], diag["cum"], diag["counts"], diag["P"]
    for i in range(order.shape[0]):
        r = row_offset + i
        g = np.asarray(gpu_col_idx[gpu_row_ptr[r]:gpu_row_ptr[r + 1]], dtype=np.int64)
        ks = int(counts[i])
        o = np.sort(order[i, :ks])
        if g.size == ks and np.array_equal(g, o):
            res["exact"] += 1
            continue
        kg = g.size
        ok = False
        if 0 < kg != ks and np.array_equal(np.sort(order[i, :kg]), g):
            if kg > ks and cum[i, kg - 2] - p <= CUT_TOL:
                ok = True
            if kg < ks and p - cum[i, kg - 1] <= CUT_TOL:
                ok = True
            if ok:
                res["excused_A"] += 1
                continue
        if kg == ks and np.all(np.diff(g) > 0) and g.min() >= 0 and g.max() < P.shape[1]:
            a = np.sort(P[i, g])[::-1]
            b = np.sort(P[i, o])[::-1]
            if np.all(np.abs(a - b) <= TIE_REL * np.maximum(a, b)):
                res["neartie_B"] += 1
                continue
        res["fail"] += 1
        if len(res["fail_rows"]) < 10:
            res["fail_rows"].append(dict(row=int(r), gpu=g.tolist()[:20], gpu_n=int(kg), oracle=o.tolist()[:20],
                                         oracle_n=ks))
    return res


def merge(a, b):
    out = dict(a)
    for k in ("exact", "excused_A", "neartie_B", "fail"):
        out[k] = a.get(k, 0) + b.get(k, 0)
    out["fail_rows"] = (a.get("fail_rows", []) + b.get("fail_rows", []))[:10]
    return out


RECORDS: list = []   # (name, payload) of this session, printed in the pytest terminal summary


def record(name: str, payload: dict):
    """Append a parity record to gpurun_out/parity.jsonl (read back for the design notes) and
    keep it for the terminal summary."""
    RECORDS.append((name, dict(payload)))
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    d = os.path.join(root, "gpurun_out")
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "parity.jsonl"), "a") as f:
        f.write(json.dumps(dict(name=name, **payload)) + "\n")
    print(f"[parity] {name}: {json.dumps(payload)}", flush=True)
