"""Benchmark of the fused attention hot path on one MI355X.

One step = one forward (fa_fwd) and one backward (fa_bwd_prep, fa_bwd_main,
fa_bwd_post) over the long-sequence workload: BNSD bf16, B=1, H=32,
S=8192, D=128, causal mask plus ALiBi bias, dO ~ N(0,1).  Inputs are
resident in HBM before the timed region.  Prints one JSON line.

Throughput counts algorithmic flops: 4*D per visible (query, key) pair for
the forward (Q K^T and P V) and 10*D for the backward (the Q K^T recompute,
dO V^T, P^T dO, dS^T Q, dS K), over the pairs the mask leaves visible.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 2.4 GHz x 4096 flop/clk (dense)
PEAK_HBM_GBS = 8000.0
METRIC = "attention fwd/bwd TFLOP/s on 1 MI355X and % of bf16 MFMA peak"
_CSRC = "tiled_attention_03_amd/csrc/"
KERNEL_SOURCES = {   # files whose text decides each timed kernel's code
    "fwd": [_CSRC + f for f in ("fa_fwd_kernel.h", "fa_fwd_bf16_d128.hip", "fa_tile.h",
                                "fa_common.h")],
    "bwd_main": [_CSRC + f for f in ("fa_bwd.hip", "fa_bwd_split.hip", "fa_tile.h", "fa_common.h")],
    "bwd_post": [_CSRC + f for f in ("fa_bwd.hip", "fa_tile.h", "fa_common.h")],
    "maxsim": [_CSRC + f for f in ("fa_maxsim.hip", "fa_tile.h", "fa_common.h")],
}
MAXSIM_METRIC = "MaxSim late-interaction scores/s on 1 MI355X and % of HBM peak"
# Algorithmic flops per visible (query, key) pair, in units of D, per timed call:
# forward Q K^T and P V; the key pass (bwd_main) recomputes Q K^T and forms
# dO V^T, P^T dO and dS^T Q; the query pass (bwd_post) adds dS K (its own
# recompute of Q K^T and dO V^T is extra work, not counted).
FLOPS_PER_PAIR_D = {"fwd": 4, "bwd_prep": 0, "bwd_main": 8, "bwd_post": 2}


def visible_pairs(pr) -> int:
    """Visible (b, h, i, j) pairs left by the workload's mask."""
    import torch
    B, H, Sq, Sk = pr.batch, pr.heads, pr.seq_q, pr.seq_k
    if Sk == 0:
        return 0
    total = 0
    for b in range(B):
        kv = pr.key_valid[b].bool() if pr.key_valid is not None else torch.ones(Sk, dtype=torch.bool)
        if pr.q_modality is None and pr.explicit_mask is None:
            if pr.causal:
                seen = kv.long().cumsum(0)          # valid keys at or before j
                total += int(seen[torch.arange(Sq).clamp(max=Sk - 1)].sum()) * H
            else:
                total += int(kv.sum()) * Sq * H
            continue
        ok = kv[None, :].expand(Sq, Sk).clone()
        if pr.causal:
            ok &= torch.ones(Sq, Sk, dtype=torch.bool).tril()
        if pr.q_modality is not None:
            allow = pr.modality_allow[pr.q_modality[b].long()][:, pr.k_modality[b].long()]
            if pr.modality_allow_diag:
                allow |= torch.eye(Sq, Sk, dtype=torch.bool)
            ok &= allow
        if pr.explicit_mask is not None:
            em = pr.explicit_mask.expand(B, H, Sq, Sk)[b]
            total += int((ok[None] & em).sum())
        else:
            total += int(ok.sum()) * H
    return total


def source_sha(paths) -> str:
    h = hashlib.sha256()
    for path in paths:
        with open(os.path.join(ROOT, path), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None
    when the counters were taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha") != source_sha(KERNEL_SOURCES[kernel]):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(pr, heads=0):
    """The plain C++ fp64 oracle timed on this host: forward + backward of the
    first ``heads`` heads (default: all of them, the whole workload), OpenMP
    over heads; plus the tiny and the causal workloads whole on a single
    thread."""
    from oracle import cpp
    threads = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)
    n = min(pr.heads, heads or pr.heads)
    sub = [t[:, :n].contiguous() for t in (pr.q, pr.k, pr.v, pr.do)]
    slopes = pr.alibi_slopes[:n].clone() if pr.alibi_slopes is not None else None
    kw = dict(causal=pr.causal, alibi_slopes=slopes, keep_prob=pr.keep_prob,
              dropout_seed=pr.dropout_seed)
    used = cpp.set_threads(min(threads, n))
    t0 = time.perf_counter()
    cpp.attention_fwd(sub[0], sub[1], sub[2], pr.scale, **kw)
    cpp.attention_bwd(*sub, pr.scale, **kw)
    dt = time.perf_counter() - t0
    pairs = n * pr.seq_q * (pr.seq_q + 1) // 2 if pr.causal else n * pr.seq_q * pr.seq_k
    flops = 14 * pr.head_dim * pairs
    # single-threaded: the tiny and the causal workloads whole
    from tiled_attention_03_amd import inputs
    cpp.set_threads(1)
    single = {}
    for cid in (1, 2):
        c = inputs.config(cid)
        s0 = time.perf_counter()
        cpp.attention_fwd(c.q, c.k, c.v, c.scale, causal=c.causal)
        cpp.attention_bwd(c.q, c.k, c.v, c.do, c.scale, causal=c.causal)
        single[c.name] = round(time.perf_counter() - s0, 4)
    cpp.set_threads(used)
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(min(threads, n)),
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": (f"fwd+bwd of all {n} heads" if n == pr.heads else
                       f"fwd+bwd of {n} of {pr.heads} heads (b=0, h<{n})") +
                      f" at S={pr.seq_q}: the plain C++ fp64 oracle, OpenMP over heads; "
                      f"algorithmic flops 14*D per visible pair",
            "single_thread_seconds": single}


def maxsim_bytes(case) -> int:
    """Bytes the MaxSim result depends on: every query row, the valid document
    rows, the document mask, and the outputs (rowmax float32, score float32)."""
    B, Lq, D = case.q.shape
    Ld = case.d.shape[1]
    valid_docs = int(case.d_valid.sum()) if case.d_valid is not None else B * Ld
    es = case.q.element_size()
    mask = B * Ld if case.d_valid is not None else 0
    return B * Lq * D * es + valid_docs * D * es + mask + B * Lq * 4 + B * 4


PEAK_FP8_TFLOPS = 5033.2       # dense fp8 MFMA: twice the bf16 rate


def bench_fp8(args):
    """The fp8 forward (pre-pass + main kernel) on the long workload's inputs,
    quantized per tensor to e4m3.  Forward only: the fp8 path has no backward."""
    import torch
    from tiled_attention_03_amd import binding as fa
    from tiled_attention_03_amd import inputs

    pr = inputs.config(args.config, with_do=False)
    dev = "cuda:0"
    (q8, qs), (k8, ks), (v8, vs) = (inputs.fp8_quantize(t) for t in (pr.q, pr.k, pr.v))
    q8, k8, v8 = q8.to(dev), k8.to(dev), v8.to(dev)
    kw = fa.problem_kwargs(pr, dev)
    o = torch.empty(q8.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(pr.batch, pr.heads, pr.seq_q, dtype=torch.float32, device=dev)
    p, keep = fa.make_problem(q8, k8, heads=pr.heads, layout=pr.layout, **kw)
    import ctypes
    n = ctypes.c_size_t(0)
    fa._check(fa.lib.fa_fwd_fp8_workspace_size(ctypes.byref(p), ctypes.byref(n)), "workspace")
    ws = torch.empty(max(n.value, 256), dtype=torch.uint8, device=dev)
    pp = ctypes.byref(p)
    stream = fa._stream()

    def call():
        fa._check(fa.lib.fa_fwd_fp8(pp, fa._ptr(q8), fa._ptr(k8), fa._ptr(v8), qs, ks, vs,
                                    fa._ptr(o), fa._ptr(lse), fa._ptr(ws), ws.numel(), stream),
                  "fa_fwd_fp8")

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    wall0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record()
        call()
        e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / args.steps
    pairs = visible_pairs(pr)
    flops = 4 * pr.head_dim * pairs
    tf = flops / (ms * 1e-3) / 1e12
    rec = {
        "metric": "attention fwd TFLOP/s with fp8 (e4m3) inputs on 1 MI355X and % of fp8 MFMA peak",
        "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3", "data": "synthetic",
        "config": {"workload": pr.name, "batch": pr.batch, "heads": pr.heads, "seq_q": pr.seq_q,
                   "seq_k": pr.seq_k, "head_dim": pr.head_dim, "layout": pr.layout,
                   "causal": pr.causal, "pse": "alibi" if pr.alibi_slopes is not None else None,
                   "pass": "fwd", "visible_pairs": pairs, "output": "bf16"},
        "wall_s_timed": round(wall, 4),
        "roofline": {"kernel": "fwd_fp8 (pre-pass + main)", "bound": "mfma", "achieved": round(tf, 2),
                     "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_FP8_TFLOPS, 4), "traffic": None,
                     "flops_per_launch": flops},
    }
    print(json.dumps(rec), flush=True)


def bench_maxsim(args):
    """The MaxSim kernel on the late-interaction workload's own tensors."""
    import torch
    from tiled_attention_03_amd import binding as fa
    from tiled_attention_03_amd import inputs

    case = inputs.maxsim_workload()
    dev = "cuda:0"
    q, d = case.q.to(dev), case.d.to(dev)
    dv = case.d_valid.to(dev)
    B, Lq, D = q.shape
    rm = torch.empty(B, Lq, dtype=torch.float32, device=dev)
    sc = torch.empty(B, dtype=torch.float32, device=dev)
    dv = fa._as_bytes(dv)                     # the mask as bytes once, outside the timed calls
    call = lambda: fa.maxsim(q, d, d_valid=dv, rowmax=rm, score=sc)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    wall0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record()
        call()
        e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / args.steps
    # cold cache: calls alternate between two copies of the inputs (2 x 214 MB, more
    # than the 256 MB Infinity Cache), so each call's inputs come from HBM
    q2, d2, dv2 = q.clone(), d.clone(), dv.clone()
    rm2, sc2 = torch.empty_like(rm), torch.empty_like(sc)
    sets = ((q, d, dv, rm, sc), (q2, d2, dv2, rm2, sc2))
    for i in range(2 * args.warmup):
        a = sets[i % 2]
        fa.maxsim(a[0], a[1], d_valid=a[2], rowmax=a[3], score=a[4])
    torch.cuda.synchronize()
    cold = 0.0
    for i, (e0, e1) in enumerate(evs):
        a = sets[i % 2]
        e0.record()
        fa.maxsim(a[0], a[1], d_valid=a[2], rowmax=a[3], score=a[4])
        e1.record()
    torch.cuda.synchronize()
    cold_ms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / args.steps
    nbytes = maxsim_bytes(case)
    gbs = nbytes / (cold_ms * 1e-3) / 1e9
    traffic = traffic_for("maxsim")
    rec = {
        "metric": MAXSIM_METRIC, "value": round(B / (ms * 1e-3), 1), "unit": "scores/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": case.name, "batch": B, "len_q": Lq, "len_d": d.shape[1],
                   "dim": D, "valid_docs": int(case.d_valid.sum())},
        "wall_s_timed": round(wall, 4),
        "cache": {"warm_ms": round(ms, 5), "cold_ms": round(cold_ms, 5),
                  "note": "value: the same inputs every call (warm); cold: calls alternate "
                          "between two input copies larger together than the Infinity Cache; "
                          "the roofline uses the cold time"},
        "roofline": {"kernel": "maxsim", "bound": "hbm", "achieved": round(gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": traffic, "bytes_per_launch": nbytes},
    }
    if not args.no_cpu_baseline:
        import oracle
        try:
            from threadpoolctl import threadpool_info
            threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
        except Exception:  # pragma: no cover - reporting only
            threads = os.cpu_count() or 1
        # the whole workload, repeated for about ten seconds
        reps, t0 = 0, time.perf_counter()
        while reps < 100 and (reps == 0 or time.perf_counter() - t0 < 10.0):
            oracle.maxsim(case.q, case.d, None, case.d_valid)
            reps += 1
        dt = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": round(reps * B / dt, 2), "unit": "scores/s",
                               "cores": int(threads), "kind": "oracle", "seconds": round(dt, 3),
                               "sample": f"the whole workload ({B} samples) x {reps}, numpy "
                                         f"float64"}
    print(json.dumps(rec), flush=True)


def attention_bytes(pr) -> int:
    """Bytes the forward result depends on: every query row, the key and value
    rows some query may see (valid keys only under a padding mask), the masks,
    and the outputs O and LSE."""
    es = pr.q.element_size()
    D, H, B = pr.head_dim, pr.heads, pr.batch
    q_bytes = B * H * pr.seq_q * D * es
    if pr.key_valid is not None:
        kv_rows = int(pr.key_valid.sum()) * H
    else:
        kv_rows = B * H * pr.seq_k
    mask_bytes = 0
    if pr.key_valid is not None:
        mask_bytes += pr.key_valid.numel()
    if pr.q_modality is not None:
        mask_bytes += pr.q_modality.numel() + pr.k_modality.numel()
    return q_bytes + 2 * kv_rows * D * es + mask_bytes + q_bytes + B * H * pr.seq_q * 4


def bench_config(cid: int, steps: int, warmup: int) -> dict:
    """Forward (and, for information, backward) times of one more workload:
    HIP events around each call on the call's stream; warm = the same tensors
    every call, cold = calls alternating between two tensor sets."""
    import torch
    from tiled_attention_03_amd import binding as fa
    from tiled_attention_03_amd import inputs

    dev = "cuda:0"
    pr = inputs.config(cid)
    kw = fa.problem_kwargs(pr, dev)
    sets = []
    for _ in range(2):
        q, k, v, do = (t.to(dev) for t in (pr.q, pr.k, pr.v, pr.do))
        o = torch.empty_like(q)
        lse = torch.empty(pr.batch, pr.heads, pr.seq_q, dtype=torch.float32, device=dev)
        sets.append((q, k, v, do, o, lse, torch.empty_like(q), torch.empty_like(k),
                     torch.empty_like(v)))
    plan = fa.Plan(sets[0][0], sets[0][1], heads=pr.heads, layout=pr.layout, **kw)

    def fwd(t):
        plan.fwd(t[0], t[1], t[2], t[4], t[5])

    def bwd(t):   # fa_bwd, the whole backward (its steps, or one pass for short query blocks)
        plan.bwd(t[0], t[1], t[2], t[4], t[5], t[3], t[6], t[7], t[8])

    def timed(fn, alternate):
        for i in range(warmup):
            fn(sets[i % 2] if alternate else sets[0])
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for i, (e0, e1) in enumerate(evs):
            t = sets[i % 2] if alternate else sets[0]
            e0.record()
            fn(t)
            e1.record()
        torch.cuda.synchronize()
        ts = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
        return ts[len(ts) // 2]

    fwd_warm, fwd_cold = timed(fwd, False), timed(fwd, True)
    for t in sets:
        fwd(t)
    bwd_warm = timed(bwd, False)
    pairs = visible_pairs(pr)
    D = pr.head_dim
    f_fwd, f_bwd = 4 * D * pairs, 10 * D * pairs
    nbytes = attention_bytes(pr)
    rec = {"workload": pr.name, "visible_pairs": pairs, "median_of": steps,
           "fwd_ms_warm": round(fwd_warm, 5), "fwd_ms_cold": round(fwd_cold, 5),
           "fwd_tflops": round(f_fwd / (fwd_warm * 1e-3) / 1e12, 2),
           "fwd_pct_of_bf16_peak": round(100 * f_fwd / (fwd_warm * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
           "fwd_bytes": nbytes,
           "fwd_gbs_cold": round(nbytes / (fwd_cold * 1e-3) / 1e9, 1),
           "fwd_pct_of_hbm_cold": round(100 * nbytes / (fwd_cold * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
           "bwd_ms_warm": round(bwd_warm, 5),
           "bwd_tflops": round(f_bwd / (bwd_warm * 1e-3) / 1e12, 2)}
    del sets, plan
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=5, help="workload id 1..5 (5 = the headline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=0,
                    help="heads in the CPU-baseline sample (0: all of them)")
    ap.add_argument("--more", default="1,2,3,4",
                    help="comma-separated workload ids whose forward is also timed and reported "
                         "under 'workloads' (empty: none)")
    ap.add_argument("--keep-prob", type=float, default=1.0,
                    help="dropout keep probability (1.0 = no dropout, the headline workload)")
    ap.add_argument("--dropout-seed", type=int, default=0x5EED)
    ap.add_argument("--workload", choices=("attention", "maxsim", "fp8"), default="attention",
                    help="attention: the fused attention step (the headline); maxsim: the "
                         "late-interaction MaxSim kernel; fp8: the forward with e4m3 inputs")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (reference for "
                         "the FETCH_SIZE / WRITE_SIZE counters) and exit")
    ap.add_argument("--workloads-only", action="store_true",
                    help="only time the --more workloads (20 calls each after 5 warm-up) and "
                         "print their records; no headline step (for profiling runs)")
    args = ap.parse_args()
    if args.workloads_only:
        print(json.dumps({"workloads": {f"c{c}": bench_config(int(c), 20, 5)
                                        for c in args.more.split(",") if c}}))
        return
    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 3}))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(every (batch, head) is independent: shard heads across GPUs and run this "
              "per GPU).", file=sys.stderr)
        sys.exit(2)

    if args.workload == "maxsim":
        bench_maxsim(args)
        return
    if args.workload == "fp8":
        bench_fp8(args)
        return

    import torch
    from tiled_attention_03_amd import binding as fa
    from tiled_attention_03_amd import inputs

    dev = "cuda:0"
    pr = inputs.config(args.config)
    pr.keep_prob, pr.dropout_seed = args.keep_prob, args.dropout_seed
    q, k, v, do = (t.to(dev) for t in (pr.q, pr.k, pr.v, pr.do))
    kw = fa.problem_kwargs(pr, dev)
    plan = fa.Plan(q, k, heads=pr.heads, layout=pr.layout, **kw)
    o = torch.empty_like(q)
    lse = torch.empty(pr.batch, pr.heads, pr.seq_q, dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    names = ("fwd", "bwd_prep", "bwd_main", "bwd_post")

    def step(ev=None):
        calls = (lambda: plan.fwd(q, k, v, o, lse),
                 lambda: plan.bwd_prep(o, do),
                 lambda: plan.bwd_main(q, k, v, lse, do, dk, dv),
                 lambda: plan.bwd_post(q, k, v, lse, do, dq))
        for n, c in enumerate(calls):
            if ev is not None:
                ev[n][0].record()
            c()
            if ev is not None:
                ev[n][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in names] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for s in range(args.steps):
        step(evs[s])
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    per = {n: sum(evs[s][i][0].elapsed_time(evs[s][i][1]) for s in range(args.steps)) / args.steps
           for i, n in enumerate(names)}

    # cold cache: steps alternate between two full sets of tensors (each set is
    # several hundred MB, beyond the 256 MB Infinity Cache)
    set_a = (q, k, v, do, o, lse, dq, dk, dv)
    set_b = tuple(t.clone() for t in set_a)

    def step_on(ts):
        q_, k_, v_, do_, o_, lse_, dq_, dk_, dv_ = ts
        plan.fwd(q_, k_, v_, o_, lse_)
        plan.bwd_prep(o_, do_)
        plan.bwd_main(q_, k_, v_, lse_, do_, dk_, dv_)
        plan.bwd_post(q_, k_, v_, lse_, do_, dq_)

    for i in range(2):
        step_on((set_a, set_b)[i % 2])
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for s in range(args.steps):
        step_on((set_a, set_b)[s % 2])
    c1.record()
    torch.cuda.synchronize()
    cold_ms = c0.elapsed_time(c1) / args.steps
    del set_b

    pairs = visible_pairs(pr)
    D = pr.head_dim
    f_fwd, f_bwd = 4 * D * pairs, 10 * D * pairs
    value = (f_fwd + f_bwd) / (ms_per_step * 1e-3) / 1e12
    fwd_tf = f_fwd / (per["fwd"] * 1e-3) / 1e12
    bwd_ms = per["bwd_prep"] + per["bwd_main"] + per["bwd_post"]
    bwd_tf = f_bwd / (bwd_ms * 1e-3) / 1e12
    dom = max(("fwd", "bwd_main", "bwd_post"), key=lambda n: per[n])
    dom_flops = FLOPS_PER_PAIR_D[dom] * D * pairs
    achieved = dom_flops / (per[dom] * 1e-3) / 1e12
    # the recorded counters were taken without dropout
    traffic = traffic_for(dom) if pr.keep_prob >= 1.0 else None
    dt = {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}[pr.dtype]
    rec = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic",
        "config": {"workload": pr.name, "batch": pr.batch, "heads": pr.heads,
                   "seq_q": pr.seq_q, "seq_k": pr.seq_k, "head_dim": D, "layout": pr.layout,
                   "causal": pr.causal, "pse": "alibi" if pr.alibi_slopes is not None else None,
                   "pass": "fwd+bwd", "visible_pairs": pairs, "keep_prob": pr.keep_prob},
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "fwd": {"ms": round(per["fwd"], 4), "tflops": round(fwd_tf, 2),
                "pct_of_bf16_peak": round(100 * fwd_tf / PEAK_BF16_TFLOPS, 2)},
        "bwd": {"ms": round(bwd_ms, 4), "tflops": round(bwd_tf, 2),
                "pct_of_bf16_peak": round(100 * bwd_tf / PEAK_BF16_TFLOPS, 2)},
        "kernel_ms": {n: round(per[n], 4) for n in names},
        "wall_s_timed": round(wall, 4),
        "cache": {"warm_ms_per_step": round(ms_per_step, 4), "cold_ms_per_step": round(cold_ms, 4),
                  "note": "value: the same tensors every step (warm); cold: steps alternate "
                          "between two tensor sets larger than the Infinity Cache"},
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "flops_per_launch": dom_flops},
        "kernel_tflops": {n: round(FLOPS_PER_PAIR_D[n] * D * pairs / (per[n] * 1e-3) / 1e12, 2)
                          for n in names if FLOPS_PER_PAIR_D[n]},
    }
    if args.more:
        rec["workloads"] = {f"c{c}": bench_config(int(c), 50, 10) for c in args.more.split(",") if c}
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(pr, heads=args.cpu_heads) if args.config == 5 else None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
