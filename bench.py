"""Benchmark: attention fwd+bwd on one MI355X, BSHD bf16, non-causal.

A step is one pass of the whole path on one batch of resident synthetic input:
    attn_fwd -> attn_bwd_preprocess -> attn_bwd
on the per-rank shard of the Wan attention layer that LightX2V PR #1234 times
("Performance": N=27280, 40 heads over 4 sequence-parallel ranks -> 10 heads,
D=128, bf16): B=1, S=27280, H=10, D=128, q/k/v/dO ~ N(0,1) rounded to bf16.

Throughput is algorithmic attention FLOPs (forward 4*B*H*S^2*D, backward 2.5x
that) over the measured step time.  Each library call is one kernel, and
hipEvents recorded around each call on the launch stream give every kernel's
average duration inside the timed region; the dominant kernel's roofline line
uses its own algorithmic FLOPs and that duration.  The fp64 CPU oracle is
timed beside it on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--graph]
(defaults: 10 warm-up and 50 timed steps; per-step median, min and mean are reported
beside the mean-based value; --graph times replays of one captured HIP graph of the step,
which removes the launch gaps that dominate the small workloads)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd+bwd TFLOP/s and % bf16 MFMA peak, Wan shard N=27280 H=10 D=128"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA (published)
# executed / algorithmic MFMA FLOPs of one fwd+bwd step: (2 + 7) / (2 + 5) products
EXECUTED_PER_ALGORITHMIC = 9.0 / 7.0
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="wan_shard",
                    help="wan_shard (the metric's workload) or another named workload: "
                         "probe_hs16, dit_s1024, mask_s4096, varlen4, wan_shard_gqa, "
                         "wan_shard_causal")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=27280,
                    help="query rows of one head in the CPU-oracle sample")
    ap.add_argument("--ring-chunks", type=int, default=0,
                    help="time the ring / context-parallel path instead: keys split into this "
                         "many chunks, per-chunk forwards merged by attn_lse_merge, per-chunk "
                         "backward with the merged statistics (attn_bwd_accum), fp32 -> bf16 casts")
    ap.add_argument("--data", default="normal", choices=("normal", "zeros"),
                    help="input values: normal (q, k, v, dO ~ N(0,1) rounded to bf16, the "
                         "benchmark's data) or zeros (same shapes and work, minimal switching "
                         "activity: shows how much of the time the power limit sets)")
    ap.add_argument("--graph", action="store_true",
                    help="time the steps as replays of one captured HIP graph of the step (the "
                         "same three kernels without per-launch gaps); per-kernel times then "
                         "come from the same number of eager steps run after the timed region")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (a known "
                         "byte count for scaling the profiler's HBM counters)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_wan_shard_hbm_traffic.json")


def kernel_source_hash():
    """Hash of the kernel sources with their // comments and blank lines removed (so that
    comment edits keep recorded counters valid); HBM counters recorded for another hash
    are stale."""
    import hashlib
    import re
    h = hashlib.sha256()
    d = os.path.join(ROOT, "attention_flash_attn_amd", "csrc")
    for f in sorted(os.listdir(d)):
        h.update(f.encode())
        with open(os.path.join(d, f), encoding="utf-8") as fh:
            code = [re.sub(r"\s*//.*$", "", line).rstrip() for line in fh]
        h.update("\n".join(line for line in code if line).encode())
    return h.hexdigest()[:16]


def recorded_traffic(workload, kernel):
    """Calibrated HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary, or None when it was taken on other kernel sources or another workload."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if workload != "wan_shard" or rec.get("source_hash") != kernel_source_hash():
        return None
    k = {"attn_fwd": "fwd", "attn_bwd": "bwd"}[kernel]
    return rec["kernels"][k]["hbm_bytes_per_launch"]


def describe(w):
    if w.name == "wan_shard":
        return (f"wan_shard: B={w.B} N={w.S} H={w.H} D={w.D}, BSHD bf16, non-causal, no mask "
                "(one Ulysses rank of the 40-head Wan layer)")
    kind = "causal (FLOPs of the S(S+1)/2 attended pairs)" if w.causal else "non-causal"
    if w.varlen:
        return f"{w.name}: packed varlen lengths {list(w.seqlens)} H={w.H} D={w.D}, bf16, {kind}"
    m = f"key mask valid lengths {list(w.valid_lens)}" if w.valid_lens else "no mask"
    kv = f" Hk={w.Hk}" if w.Hk is not None else ""
    return f"{w.name}: B={w.B} S={w.S} H={w.H}{kv} D={w.D}, BSHD bf16, {kind}, {m}"


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_head_tflops(t, b, h, rows, D):
    """fp64 oracle on head (b, h): the first `rows` query rows against all keys, forward,
    delta, dQ of those rows and their full dK/dV contribution (same per-row work as the
    full problem).  Returns (TFLOP/s at the algorithmic count, seconds)."""
    import oracle
    from attention_flash_attn_amd import inputs as I

    q, k, v, do = (I.f64_from_bf16_bits(x[b:b + 1, :, h:h + 1]) for x in (t.q, t.k, t.v, t.do))
    q, do = q[:, :rows], do[:, :rows]
    t0 = time.perf_counter()
    out, lse = oracle.attn_fwd(q, k, v)
    oracle.attn_bwd(q, k, v, out, lse, do)
    dt = time.perf_counter() - t0
    return 3.5 * 4.0 * rows * k.shape[1] * D / dt / 1e12, dt


def cpu_baseline(w, t, rows):
    """The oracle on all host threads over one head of the workload, plus a one-thread
    run over one head of the 1024-token DiT workload for a per-core figure."""
    import oracle
    from attention_flash_attn_amd import inputs as I

    cores = oracle.num_threads()
    value, dt = oracle_head_tflops(t, 0, 0, rows, w.D)
    small = I.WORKLOADS["dit_s1024"]
    oracle.set_num_threads(1)
    try:
        v1, dt1 = oracle_head_tflops(I.draw_workload(small), 0, 0, small.S, small.D)
    finally:
        oracle.set_num_threads(cores)
    return {"value": value, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"one head (b=0,h=0), {rows} of {w.S} query rows x all {w.S} keys, "
                      f"fwd+delta+dQ+dK/dV in fp64, {dt:.1f} s on {cores} threads of {cpu_model()}",
            "per_core": {"value": v1, "unit": "TFLOP/s", "cores": 1,
                         "sample": f"one head of dit_s1024 (S={small.S}, D={small.D}), same passes, "
                                   f"{dt1:.2f} s on 1 thread"}}


def calibration_copy(mb):
    """One plain device copy of `mb` MiB after the timed work: a known byte count that
    scales the profiler's HBM counters."""
    if mb <= 0:
        return {}
    import torch
    n = mb << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    return {"copy_calibration_bytes": n}


def run_ring(args, w, t, C):
    """The ring / context-parallel path on one GPU: the workload's keys in C chunks."""
    import numpy as np
    import torch

    import attention_flash_attn_amd as A

    if w.varlen or w.causal or w.Hk is not None:
        raise SystemExit("--ring-chunks applies to dense non-causal multi-head workloads")
    dev = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v, do = (dev(x) for x in (t.q, t.k, t.v, t.do))
    B, S, H, D = w.B, w.S, w.H, w.D
    bounds = [(c * S // C, (c + 1) * S // C) for c in range(C)]
    mask = None if t.key_mask is None else torch.from_numpy(t.key_mask).cuda()
    ks = [k[:, a:b].contiguous() for a, b in bounds]
    vs = [v[:, a:b].contiguous() for a, b in bounds]
    ms = [None if mask is None else mask[:, a:b].contiguous() for a, b in bounds]
    outs = [torch.empty_like(q) for _ in bounds]
    lses = [torch.empty((B, H, S), dtype=torch.float32, device="cuda") for _ in bounds]
    out, lse = torch.empty_like(q), torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    delta = torch.empty_like(lse)
    dq_acc = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    dk_acc = [torch.empty(x.shape, dtype=torch.float32, device="cuda") for x in ks]
    dv_acc = [torch.empty(x.shape, dtype=torch.float32, device="cuda") for x in vs]
    dq = torch.empty_like(q)
    dks, dvs = [torch.empty_like(x) for x in ks], [torch.empty_like(x) for x in vs]

    def step(ev=None):
        rec = (lambda i: ev[i].record()) if ev is not None else (lambda i: None)
        rec(0)
        for c in range(C):
            A.attn_fwd(q, ks[c], vs[c], ms[c], None, out=outs[c], lse=lses[c])
        rec(1)
        A.attn_lse_merge(outs, lses, out=out, lse=lse)
        rec(2)
        A.attn_bwd_preprocess(out, do, delta=delta)
        rec(3)
        for c in range(C):
            A.attn_bwd_accum(q, ks[c], vs[c], lse, delta, do, dq_acc, dk_acc[c], dv_acc[c], ms[c],
                             add_dq=c > 0, add_dkdv=False)
        rec(4)
        A.attn_cast_bf16(dq_acc, dq)
        for c in range(C):
            A.attn_cast_bf16(dk_acc[c], dks[c])
            A.attn_cast_bf16(dv_acc[c], dvs[c])
        rec(5)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        step(evs[i])
    torch.cuda.synchronize()
    per = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(5)] for e in evs])
    step_ms = float(evs[0][0].elapsed_time(evs[-1][5])) / K
    fwd_ms, merge_ms, pre_ms, bwd_ms, cast_ms = (float(x) for x in np.median(per, 0))
    f_fwd = w.fwd_flops()
    total = 3.5 * f_fwd
    rows = B * S * H
    merge_bytes = C * (rows * D * 2 + rows * 4) + rows * D * 2 + rows * 4
    merge_gbs = merge_bytes / (merge_ms * 1e-3) / 1e9
    return {
        "metric": f"attention fwd+bwd TFLOP/s, ring path with the keys in {C} chunks",
        "value": round(total / (step_ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": describe(w) + f"; keys in {C} equal chunks", "chunks": C},
        "kernels_ms_median": {"attn_fwd x%d" % C: round(fwd_ms, 4), "attn_lse_merge": round(merge_ms, 4),
                              "attn_bwd_preprocess": round(pre_ms, 4),
                              "attn_bwd_accum x%d" % C: round(bwd_ms, 4),
                              "attn_cast_bf16 x%d" % (2 * C + 1): round(cast_ms, 4)},
        "merge_roofline": {"bound": "hbm", "achieved": round(merge_gbs, 1), "peak": PEAK_HBM_GBS,
                           "unit": "GB/s", "frac": round(merge_gbs / PEAK_HBM_GBS, 4),
                           "traffic": None, "bytes_per_launch": merge_bytes},
    }


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the attention path here has no multi-GPU "
              "mode (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import attention_flash_attn_amd as A
    from attention_flash_attn_amd import inputs as I

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    A.lib()
    w = I.WORKLOADS[args.workload]
    t = I.draw_workload(w)
    if args.data == "zeros":
        import dataclasses
        t = dataclasses.replace(t, **{n: np.zeros_like(getattr(t, n)) for n in ("q", "k", "v", "do")})
    if args.ring_chunks > 0:
        res = run_ring(args, w, t, args.ring_chunks)
        res.update(calibration_copy(args.copy_calibration_mb))
        print(json.dumps(res), flush=True)
        return
    dev = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v, do = (dev(x) for x in (t.q, t.k, t.v, t.do))
    B, S, H, D = w.B, w.S, w.H, w.D
    out = torch.empty_like(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    mask = None if t.key_mask is None else torch.from_numpy(t.key_mask).cuda()
    if w.varlen:
        T = w.T
        lse = torch.empty((H, T), dtype=torch.float32, device="cuda")
        delta = torch.empty((1, H, T), dtype=torch.float32, device="cuda")
        cu_host = torch.from_numpy(t.cu_seqlens)
        cu_dev = cu_host.cuda()

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        if w.varlen:
            A.attn_varlen_fwd(q, k, v, (cu_host, cu_dev), None, out=out, lse=lse, causal=w.causal)
        else:
            A.attn_fwd(q, k, v, mask, None, out=out, lse=lse, causal=w.causal)
        if ev is not None:
            ev[1].record()
        A.attn_bwd_preprocess(out, do, delta=delta)
        if ev is not None:
            ev[2].record()
        if w.varlen:
            A.attn_varlen_bwd(q, k, v, lse, delta, do, (cu_host, cu_dev), None, dq=dq, dk=dk, dv=dv,
                              causal=w.causal)
        else:
            A.attn_bwd(q, k, v, lse, delta, do, mask, None, dq=dq, dk=dk, dv=dv, causal=w.causal)
        if ev is not None:
            ev[3].record()

    if not w.varlen:
        lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
        delta = torch.empty_like(lse)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    graph_ms = None
    if args.graph:
        # One step captured as a HIP graph (every output buffer preallocated, no memset in
        # the captured calls), warmed up, then K replays timed between two events.
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            step()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        g0.record()
        for _ in range(K):
            g.replay()
        g1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        graph_ms = g0.elapsed_time(g1) / K
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    torch.cuda.synchronize()
    t0e = time.perf_counter()
    for i in range(K):
        step(evs[i])
    torch.cuda.synchronize()
    if graph_ms is None:
        wall = time.perf_counter() - t0e
    per = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3])]
                    for e in evs])  # ms
    steps_each = np.array([e[0].elapsed_time(e[3]) for e in evs])
    eager_ms = float(evs[0][0].elapsed_time(evs[-1][3])) / K
    step_ms = graph_ms if graph_ms is not None else eager_ms
    fwd_ms, pre_ms, bwd_ms = (float(x) for x in per.mean(0))

    f_fwd = w.fwd_flops()
    f_bwd = 2.5 * f_fwd
    total = f_fwd + f_bwd
    value = total / (step_ms / 1e3) / 1e12
    kernels = {"attn_fwd": (fwd_ms, f_fwd), "attn_bwd": (bwd_ms, f_bwd)}
    dom = max(kernels, key=lambda n: kernels[n][0])
    dom_ms, dom_flops = kernels[dom]
    achieved = dom_flops / (dom_ms / 1e3) / 1e12
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": (f"synthetic: q,k,v,dO ~ N(0,1) seed {w.seed}, rounded to bf16" if args.data == "normal"
                 else "synthetic: q,k,v,dO all zero (power-limit diagnostic, not the metric's data)"),
        "config": {"workload": describe(w), "batch": B, "seq_len": S, "heads": H,
                   "head_dim": D, "parallelism": "none"},
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        # MFMA work as executed: the forward's 2 products and the backward's 7 (dK/dV: 4,
        # dQ: 3, of which 2 recompute S and dP), against the 5 the algorithmic count credits
        "executed_tflops": round(EXECUTED_PER_ALGORITHMIC * value, 2),
        "pct_bf16_peak_executed": round(100 * EXECUTED_PER_ALGORITHMIC * value / PEAK_BF16_TFLOPS, 2),
        "kernels_ms": {"attn_fwd": round(fwd_ms, 4), "attn_bwd_preprocess": round(pre_ms, 4),
                       "attn_bwd": round(bwd_ms, 4)},
        "fwd_tflops": round(f_fwd / (fwd_ms / 1e3) / 1e12, 2),
        "bwd_tflops": round(f_bwd / (bwd_ms / 1e3) / 1e12, 2),
        "wall_ms_per_step": round(1e3 * wall / K, 4),
        "step_ms_stats": {"median": round(float(np.median(steps_each)), 4),
                          "min": round(float(steps_each.min()), 4),
                          "mean": round(float(steps_each.mean()), 4)},
        "kernels_ms_median": {"attn_fwd": round(float(np.median(per[:, 0])), 4),
                              "attn_bwd_preprocess": round(float(np.median(per[:, 1])), 4),
                              "attn_bwd": round(float(np.median(per[:, 2])), 4)},
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic(w.name, dom)},
    }
    if graph_ms is not None:
        res["step_mode"] = "hip graph replay (kernels_ms, step_ms_stats: eager steps)"
        res["eager_ms_per_step"] = round(eager_ms, 4)
    res.update(calibration_copy(args.copy_calibration_mb))
    if not args.no_cpu_baseline and not w.varlen and w.valid_lens is None and not w.causal:
        res["cpu_baseline"] = cpu_baseline(w, t, min(args.cpu_rows, w.S))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
