#!/usr/bin/env python3
"""Benchmark of the Top-p block-sparse attention hot path on one MI355X.

One step = one layer: Top-p routing (pool, score/softmax/cut, CSR) + the attention plan
(work list, V transpose) + block-sparse attention, over a synthetic bf16 layer that is
already resident in HBM.  Default workload: Wan2.1-14B-shaped layer, H=40, N=32760
(21x30x52 latent tokens), d=128, 64-token blocks, p=0.9.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E
SCHEDULES = ("lpt", "identity", "head_lpt", "xcd", "rlb", "head_desc")
METRIC = "sparse-attn effective TFLOP/s (executed blocks) + ms/layer at N=32760 H=40 d=128"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def executed_flops(row_ptr, col_idx, N, nqb, block_q, block_k, d):
    """Sum over kept (query block, key block) pairs of 4*|q block|*|k block|*d (ragged sizes)."""
    import numpy as np
    rows = row_ptr.size - 1
    cnt = np.diff(row_ptr)
    i = np.arange(rows) % nqb
    qlen = np.minimum(block_q, N - i * block_q).astype(np.float64)
    klen = np.minimum(block_k, N - col_idx.astype(np.int64) * block_k).astype(np.float64)
    per_row_k = np.add.reduceat(klen, row_ptr[:-1]) if klen.size else np.zeros(rows)
    per_row_k = np.where(cnt > 0, per_row_k, 0.0)
    return float(4.0 * d * np.sum(qlen * per_row_k)), float(4.0 * d * block_q * block_k * cnt.sum())


def cu_balance(trace_np):
    """max/mean over CUs of busy time (union of the tile intervals run on each CU)."""
    import numpy as np
    trace_np = trace_np[trace_np[:, 2] > 0]           # records that were written
    hw = trace_np[:, 0]
    key = ((hw >> 32) << 8) | ((hw >> 8) & 0xFF)       # (XCC id, SE/SH/CU id bits of HW_ID)
    t0, t1 = trace_np[:, 1].astype(np.int64), trace_np[:, 2].astype(np.int64)
    busy = {}
    for kk in np.unique(key):
        m = key == kk
        iv = sorted(zip(t0[m].tolist(), t1[m].tolist()))
        tot, cs, ce = 0, iv[0][0], iv[0][1]
        for s, e in iv[1:]:
            if s > ce:
                tot += ce - cs
                cs, ce = s, e
            else:
                ce = max(ce, e)
        busy[int(kk)] = tot + ce - cs
    b = np.array(list(busy.values()), dtype=np.float64)
    span = (t1.max() - t0.min()) / 100.0   # 100 MHz clock -> us
    return dict(max_over_mean=float(b.max() / b.mean()), cus=int(b.size), span_us=float(span),
                mean_busy_us=float(b.mean() / 100.0))


def cpu_baseline(w, p, q, k, v, budget_s):
    """The fp64 oracle as it stands, on a bounded sample of the same layer, scaled to the
    whole layer by executed FLOP; returns the layer-equivalent effective TFLOP/s."""
    import numpy as np
    import oracle
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max((i.get("num_threads", 1) for i in info), default=1)
    except Exception:  # pragma: no cover
        threads = None
    cores = len(os.sched_getaffinity(0))
    heads = [0, w.H // 2]
    t = time.perf_counter()
    kept_per_head = {}
    for h in heads:
        kept_per_head[h], _ = oracle.route_head(q[0, h], k[0, h], w.block_q, w.block_k, p)
    t_route_head = (time.perf_counter() - t) / len(heads)
    rng = np.random.default_rng(5)
    flop_s, t_att, nrows = 0.0, 0.0, 0
    t_end = time.perf_counter() + budget_s
    while time.perf_counter() < t_end or nrows < 8:
        h = heads[nrows % len(heads)]
        i = int(rng.integers(0, w.nqb))
        kept = kept_per_head[h][i]
        qlen = min(w.block_q, w.N - i * w.block_q)
        klen = sum(min(w.block_k, w.N - j * w.block_k) for j in kept)
        t = time.perf_counter()
        oracle.sparse_attention_rows(q[0, h], k[0, h], v[0, h], w.block_q, w.block_k, {i: kept})
        t_att += time.perf_counter() - t
        flop_s += 4.0 * w.d * qlen * klen
        nrows += 1
        if nrows >= 4000:
            break
    return dict(t_route_head=t_route_head, attn_flops_per_s=flop_s / t_att, rows=nrows, heads=len(heads),
                cores=cores, threads=threads, seconds=t_route_head * len(heads) + t_att)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wan14b_n32760")
    ap.add_argument("--p", type=float, default=None)
    ap.add_argument("--schedule", default="head_desc", choices=sorted(SCHEDULES),
                    help="attention work order (the library default is head_desc: heads heaviest first)")
    ap.add_argument("--alt-p", type=float, default=0.95,
                    help="also time the layer at this p (the workload's second threshold); 0: off")
    ap.add_argument("--out", default="bf16", choices=["f32", "bf16"],
                    help="output dtype of the attention: bf16 (the layer's output, rounded to nearest even) or "
                         "f32 (accumulator precision)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip trace/copy-bandwidth extras (profiling runs)")
    ap.add_argument("--mode", default="topp", choices=["topp", "topk"], help="routing variant (default Top-p)")
    ap.add_argument("--topk", type=int, default=0, help="blocks per row for --mode topk")
    ap.add_argument("--k-min", type=int, default=1, help="lower clamp of the Top-p count")
    ap.add_argument("--k-max", type=int, default=0, help="upper clamp of the Top-p count (0: none)")
    ap.add_argument("--window", type=int, default=0, help="local window of key blocks kept around each query block")
    ap.add_argument("--sasa-groups", type=int, default=0, help="SASA over this many head groups (0: off)")
    ap.add_argument("--sasa-alpha", type=float, default=0.5, help="SASA augmentation coefficient")
    ap.add_argument("--sasa-tau", type=float, default=0.0, help="SASA trigger threshold")
    ap.add_argument("--route-every", type=int, default=1,
                    help="route on every K-th step only and reuse the CSR in between (lazy refresh of the "
                         "sparse pattern across diffusion steps; 1: route every step)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps(dict(error="this benchmark runs on one GPU: the hot path is measured on one GPU's "
                                    "share; multi-GPU runs are not supported", n_gpus=args.gpus)))
        sys.exit(2)

    import numpy as np
    import torch

    import top_block_sparse_pooled_amd as fv
    import workloads

    w = workloads.get(args.workload)
    p = args.p if args.p is not None else w.ps[0]
    dev = torch.device("cuda:0")
    log(f"[bench] generating {w.name}: H={w.H} N={w.N} d={w.d} bq={w.block_q} bk={w.block_k} p={p}")
    t = time.perf_counter()
    q, k, v = workloads.make_qkv(w)
    log(f"[bench] inputs generated in {time.perf_counter() - t:.1f}s; uploading")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    qd, kd, vd = (torch.from_numpy(a).to(tdt).to(dev).contiguous() for a in (q, k, v))
    out_dtype = torch.float32 if args.out == "f32" else None

    csr = fv.Csr.empty(1, w.H, w.N, w.block_q, w.block_k, dev)
    rws = torch.empty(fv.route_ws_bytes(1, w.H, w.N, w.d, w.block_q, w.block_k), dtype=torch.uint8, device=dev)
    aws = fv.attn_ws(qd, csr)
    o = torch.empty(qd.shape, dtype=out_dtype or tdt, device=dev)

    variant = dict(mode=args.mode, topk=args.topk, k_min=args.k_min, k_max=args.k_max, window=args.window)
    sws = None
    if args.sasa_groups > 0:
        sws = torch.empty(fv.lib().fvattn_route_sasa_ws_bytes(1, w.H, w.N, w.d, w.block_q, w.block_k,
                                                               args.sasa_groups), dtype=torch.uint8, device=dev)
    if args.mode == "topk" and args.topk < 1:
        raise SystemExit("--mode topk needs --topk >= 1")

    if args.route_every < 1:
        raise SystemExit("--route-every needs K >= 1")

    def step(ev=None, do_route=True):
        if ev is not None:
            ev[0].record()
        if not do_route:
            pass   # the CSR of the last refresh is reused; the plan is rebuilt (it may hold a copy of v)
        elif args.sasa_groups > 0:
            fv.route_sasa(qd, kd, w.block_q, w.block_k, p, groups=args.sasa_groups, alpha=args.sasa_alpha,
                          tau=args.sasa_tau, csr=csr, ws=sws, **variant)
        else:
            fv.route(qd, kd, w.block_q, w.block_k, p, csr=csr, ws=rws, **variant)
        if ev is not None:
            ev[1].record()
        fv.attn_plan(vd, csr, aws, args.schedule)
        if ev is not None:
            ev[2].record()
        fv.attn_run(qd, kd, vd, csr, aws, out=o, out_dtype=out_dtype)
        if ev is not None:
            ev[3].record()

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    routed = [i % args.route_every == 0 for i in range(args.steps)]
    for i in range(args.steps):
        step(evs[i], routed[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = 1e3 * wall / args.steps
    route_ms = float(np.mean([e[0].elapsed_time(e[1]) for e, r in zip(evs, routed) if r]))
    plan_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    attn_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))

    rp = csr.row_ptr.cpu().numpy().astype(np.int64)
    nnz = int(rp[-1])
    ci = csr.col_idx[:nnz].cpu().numpy().astype(np.int64)
    flops, flops_nominal = executed_flops(rp, ci, w.N, w.nqb, w.block_q, w.block_k, w.d)
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    value = flops / (ms_step * 1e-3) / 1e12
    elem = 2 if w.dtype == "bf16" else 4
    route_bytes = 2 * w.H * w.N * w.d * elem + 4 * (w.rows + 1) + 4 * nnz + 4 * w.H
    route_gbps = route_bytes / (route_ms * 1e-3) / 1e9
    log(f"[bench] ms/step {ms_step:.3f} (route {route_ms:.3f}, plan {plan_ms:.3f}, attn {attn_ms:.3f}); "
        f"attn {attn_tflops:.1f} TFLOP/s; route {route_gbps:.0f} GB/s; kept {nnz / (w.rows * w.nkb):.4f}")

    alt = None
    if args.alt_p and args.alt_p != p and args.mode == "topp" and args.sasa_groups == 0 and args.route_every == 1:
        # the same layer at the workload's other threshold (a few timed steps, after the main timing)
        ev2 = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(5)]
        csr2 = fv.Csr.empty(1, w.H, w.N, w.block_q, w.block_k, dev)

        def step2(ev):
            ev[0].record()
            fv.route(qd, kd, w.block_q, w.block_k, args.alt_p, csr=csr2, ws=rws, **variant)
            ev[1].record()
            fv.attn_plan(vd, csr2, aws, args.schedule)
            ev[2].record()
            fv.attn_run(qd, kd, vd, csr2, aws, out=o, out_dtype=out_dtype)
            ev[3].record()

        step2(ev2[0])
        torch.cuda.synchronize()
        for e in ev2:
            step2(e)
        torch.cuda.synchronize()
        rp2 = csr2.row_ptr.cpu().numpy().astype(np.int64)
        ci2 = csr2.col_idx[: int(rp2[-1])].cpu().numpy().astype(np.int64)
        fl2, _ = executed_flops(rp2, ci2, w.N, w.nqb, w.block_q, w.block_k, w.d)
        ms = [e[0].elapsed_time(e[3]) for e in ev2]
        a_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in ev2]))
        alt = dict(p=args.alt_p, ms_per_layer=float(np.mean(ms)), route_ms=float(np.mean([e[0].elapsed_time(e[1])
                                                                                          for e in ev2])),
                   attn_ms=a_ms, attn_tflops=fl2 / (a_ms * 1e-3) / 1e12, executed_tflop=fl2 / 1e12,
                   kept_frac=float(rp2[-1]) / (w.rows * w.nkb), steps=len(ev2))
        log(f"[bench] p={args.alt_p}: {json.dumps(alt)}")
        del csr2

    sasa_info = None
    if args.sasa_groups > 0:
        R = args.sasa_groups
        after = csr.head_load.cpu().numpy().astype(np.int64)
        base = fv.route(qd, kd, w.block_q, w.block_k, p, **variant).head_load.cpu().numpy().astype(np.int64)
        grp = np.arange(w.H) * R // w.H
        Lb = np.bincount(grp, weights=base, minlength=R)
        La = np.bincount(grp, weights=after, minlength=R)
        sasa_info = dict(groups=R, alpha=args.sasa_alpha, tau=args.sasa_tau, added=int(after.sum() - base.sum()),
                         group_load_before=[int(x) for x in Lb], group_load_after=[int(x) for x in La],
                         max_over_mean_before=float(Lb.max() / Lb.mean()),
                         max_over_mean_after=float(La.max() / La.mean()))
        log(f"[bench] sasa {json.dumps(sasa_info)}")

    traffic = None
    prof = os.path.join(ROOT, "profiles", f"attn_counters_{w.name}.json")
    if os.path.exists(prof):
        try:
            pc = json.load(open(prof))
            same = (pc.get("kernel_source_sha") == _attn_source_sha() and pc.get("p") == p
                    and pc.get("schedule") == args.schedule and pc.get("out", "f32") == args.out and pc.get("routing", "topp") == "topp"
                    and args.mode == "topp" and args.k_min == 1 and args.k_max == 0 and args.window == 0
                    and args.sasa_groups == 0)
            if same:
                traffic = pc.get("bytes_per_launch")
        except Exception:
            traffic = None

    extras = {}
    if not args.no_extras:
        bal = {}
        for sched in SCHEDULES:
            tr = torch.zeros(w.rows * 4, dtype=torch.int64, device=dev)
            fv.attn_plan(vd, csr, aws, sched)
            fv.attn_run(qd, kd, vd, csr, aws, out=o, out_dtype=out_dtype, trace=tr)
            torch.cuda.synchronize()
            bal[sched] = cu_balance(tr.cpu().numpy().reshape(-1, 4).view(np.uint64))
        extras["cu_busy"] = bal
        n = 1 << 28   # 1 GiB of fp32
        a = torch.empty(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        extras["copy_gbps"] = 5 * 2 * 4 * n / (e0.elapsed_time(e1) * 1e-3) / 1e9
        del a, b
        hl = csr.head_load.cpu().numpy().astype(np.float64)
        extras["head_load_max_over_mean"] = float(hl.max() / hl.mean())
        extras["head_kept_frac_range"] = [float(hl.min() / (w.nqb * w.nkb)), float(hl.max() / (w.nqb * w.nkb))]
        log(f"[bench] extras {json.dumps(extras)}")

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline (oracle) ~{args.cpu_seconds:.0f}s sample")
        cb = cpu_baseline(w, p, q, k, v, args.cpu_seconds)
        cpu_time = cb["t_route_head"] * w.H + flops / cb["attn_flops_per_s"]
        cpu = dict(value=flops / cpu_time / 1e12, unit="TFLOP/s", cores=cb["threads"] or cb["cores"],
                   kind="oracle",
                   sample=(f"fp64 numpy oracle on the host: routing of {cb['heads']} of {w.H} heads and exact "
                           f"attention of {cb['rows']} sampled query blocks ({cb['seconds']:.1f}s); scaled to "
                           f"the whole layer by head count and executed FLOP; "
                           f"{cb['cores']} cores visible, {cb['threads']} BLAS threads"),
                   ms_per_layer=1e3 * cpu_time)
        log(f"[bench] cpu {json.dumps(cpu)}")

    rec = dict(
        metric=METRIC, value=value, unit="TFLOP/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=ms_step, higher_is_better=True, scaling="weak", vs_baseline=None, dtype=w.dtype,
        data="synthetic",
        config=dict(workload=w.name, B=1, H=w.H, N=w.N, d=w.d, block_q=w.block_q, block_k=w.block_k, p=p,
                    routing=(variant if (args.mode != "topp" or args.k_min != 1 or args.k_max or args.window)
                             else "topp"),
                    sasa=sasa_info, route_every=args.route_every,
                    schedule=args.schedule, out=args.out, nnz=nnz, kept_frac=nnz / (w.rows * w.nkb),
                    executed_tflop=flops / 1e12, nominal_tflop=flops_nominal / 1e12),
        stages_ms=dict(route=route_ms, plan=plan_ms, attn=attn_ms),
        roofline=dict(bound="mfma", kernel=attn_kernel_name(w), achieved=attn_tflops, peak=PEAK_BF16_TFLOPS,
                      unit="TFLOP/s", frac=attn_tflops / PEAK_BF16_TFLOPS, traffic=traffic),
        routing=dict(bound="hbm", achieved=route_gbps, peak=PEAK_HBM_GBPS, unit="GB/s",
                     frac=route_gbps / PEAK_HBM_GBPS, algorithmic_bytes=route_bytes, us=1e3 * route_ms),
        cpu_baseline=cpu,
        layer_alt_p=alt,
        **extras,
    )
    print(json.dumps(rec), flush=True)


def attn_kernel_name(w):
    """The attention kernel the library runs for this workload (bf16: two wave groups per
    unit over 64-key tiles of one or two key blocks)."""
    return "k_attn_pp" if w.dtype == "bf16" else "k_attn_f32"


def _attn_source_sha():
    import hashlib
    with open(os.path.join(ROOT, "top_block_sparse_pooled_amd", "csrc", "attn.hip"), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


if __name__ == "__main__":
    main()
