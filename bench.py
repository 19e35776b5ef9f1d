#!/usr/bin/env python3
"""Benchmark of the HSTU attention hot path on one MI355X.

One step = one forward (pointwise aggregated attention + LayerNorm(AV)*U
gate, saving O and the row statistics) and one backward (dQ, dK, dV, dU,
drab_p, drab_t) over the jagged batch at N_max = 8192: B = 8 sequences with
Stochastic-Length lengths (alpha 1.6, n = 8192), H = 4 heads, d = 128, bf16
storage, seeded synthetic inputs resident in HBM before timing starts.

Throughput is algorithmic causal TFLOP/s: forward 4*d flops per causal
(query, key) pair per head, backward 8*d (four products), i.e.
2*H*d*sum L(L+1) and twice that.  Per-kernel durations come from HIP events
recorded on the launch stream around each kernel (libhstu's profiling
hooks), over the same timed steps.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=2048,
                    help="prefix length per sequence for the oracle's timed sample")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (a known-size kernel that "
                         "calibrates HBM byte counters in a profiler run)")
    return ap.parse_args()


def causal_pairs_sum(lengths):
    L = np.asarray(lengths, np.float64)
    return float((L * (L + 1)).sum())   # = 2 * causal pairs per head


def cpu_baseline(w, prefix):
    """Time the fp64 oracle (forward + epilogue + backward) on the same
    workload's sequences cut to their first `prefix` tokens."""
    import oracle
    import synth
    lens = np.minimum(w.lengths, prefix)
    idx = np.concatenate([np.arange(w.offsets[b], w.offsets[b] + lens[b]) for b in range(w.batch)])
    off = synth.offsets_of(lens)
    q, k, v, u, dg, ts = (a[idx] for a in (w.q, w.k, w.v, w.u, w.dg, w.ts))
    t0 = time.perf_counter()
    O = oracle.attn_fwd(off, ts, q, k, v, w.rab_p, w.rab_t, w.n_max)
    oracle.ln_gate(O, u, w.ln_eps)
    oracle.attn_bwd(off, ts, q, k, v, w.rab_p, w.rab_t, w.n_max, u, w.ln_eps, dg)
    dt = time.perf_counter() - t0
    flops = 3 * 2 * w.heads * w.d * causal_pairs_sum(lens)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": "fwd+LN gate+bwd of the same 8 sequences cut to their first %d tokens (T=%d, %.1f GFLOP "
                      "algorithmic, %.1f s)" % (prefix, int(lens.sum()), flops / 1e9, dt),
            "seconds": dt}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only; --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    import hstu_sequential_transducer_amd as hs

    dev = torch.device("cuda:0")
    w = synth.attn_8k(with_grad=True)
    T, H, d, F = w.total, w.heads, w.d, w.heads * w.d

    def act(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev).to(torch.bfloat16)

    q, k, v = (act(a).reshape(T, H, d) for a in (w.q, w.k, w.v))
    u, dg = act(w.u), act(w.dg)
    off = torch.from_numpy(w.offsets.astype(np.int32)).to(dev)
    ts = torch.from_numpy(w.ts.astype(np.int64)).to(dev)
    rp = torch.from_numpy(w.rab_p).to(dev)
    rt = torch.from_numpy(w.rab_t).to(dev)
    out = torch.empty((T, F), dtype=torch.bfloat16, device=dev)
    osv = torch.empty((T, F), dtype=torch.float32, device=dev)
    lst = torch.empty((T, 2), dtype=torch.float32, device=dev)

    def step():
        hs.attn_fwd(off, T, ts, q, k, v, rp, rt, w.n_max, u=u, eps=w.ln_eps, out=out, o_save=osv, ln_stats=lst)
        return hs.attn_bwd(off, T, ts, q, k, v, rp, rt, w.n_max, dg, u=u, o_save=osv, ln_stats=lst, eps=w.ln_eps)

    for _ in range(args.warmup):
        g = step()
    torch.cuda.synchronize()
    hs.profile_collect()           # drop anything recorded so far
    hs.profile_enable(True)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        g = step()
    e1.record()
    torch.cuda.synchronize()
    hs.profile_enable(False)
    kt = hs.profile_collect()
    ms = e0.elapsed_time(e1) / args.steps
    if not all(bool(torch.isfinite(g[n]).all()) for n in ("dq", "dk", "dv", "du", "drab_p", "drab_t")):
        print("bench.py: non-finite gradients", file=sys.stderr)
        sys.exit(1)

    S2 = causal_pairs_sum(w.lengths)
    f_fwd = 2.0 * H * d * S2
    f_bwd = 2.0 * f_fwd
    tflops = (f_fwd + f_bwd) / (ms * 1e-3) / 1e12
    per_kernel = {n: {"launches": c, "avg_ms": t / max(c, 1)} for n, (c, t) in kt.items()}
    # dominant kernel: the largest share of the timed region
    dom = max(kt.items(), key=lambda kv: kv[1][1])[0]
    dom_flops = {"attn_bwd_bf16_kernel": f_bwd, "attn_fwd_bf16_kernel": f_fwd}.get(dom)
    avg = per_kernel[dom]["avg_ms"]
    roof = None
    if dom_flops is not None:
        ach = dom_flops / (avg * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                "avg_ms": round(avg, 4), "algorithmic_flops_per_launch": dom_flops}
    fwd_ms = per_kernel.get("attn_fwd_bf16_kernel", {}).get("avg_ms")
    bwd_ms = per_kernel.get("attn_bwd_bf16_kernel", {}).get("avg_ms")
    res = {
        "metric": "HSTU attention fwd+bwd TFLOP/s & % MFMA peak, jagged N_max=8192",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "pct_mfma_peak": round(100.0 * tflops / MFMA_BF16_PEAK_TFLOPS, 2),
        "config": {"workload": "attn-8k-B8-SL1.6 fwd+bwd (LayerNorm(AV)*U epilogue)", "batch": w.batch,
                   "n_max": w.n_max, "heads": H, "d": d, "tokens": T, "lengths": [int(x) for x in w.lengths],
                   "fwd_gflop": round(f_fwd / 1e9, 2), "bwd_gflop": round(f_bwd / 1e9, 2), "seed": 2},
        "tokens_per_s": round(T / (ms * 1e-3), 1),
        "roofline": roof,
        "kernels": per_kernel,
        "attn_fwd_tflops": round(f_fwd / (fwd_ms * 1e-3) / 1e12, 2) if fwd_ms else None,
        "attn_bwd_tflops": round(f_bwd / (bwd_ms * 1e-3) / 1e12, 2) if bwd_ms else None,
    }
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_probe_bytes_each_way"] = n * 4
    if not args.no_cpu_baseline:
        cb = cpu_baseline(w, args.cpu_sample_tokens)
        res["cpu_baseline"] = {k2: (round(v2, 6) if isinstance(v2, float) else v2) for k2, v2 in cb.items()}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
