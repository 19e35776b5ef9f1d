#!/usr/bin/env python3
"""Benchmark of the HSTU attention hot path on one MI355X.

One step = one forward (pointwise aggregated attention + LayerNorm(AV)*U
gate, saving O and the row statistics) and one backward (dQ, dK, dV, dU,
drab_p, drab_t) over the jagged batch at N_max = 8192: B = 8 sequences with
Stochastic-Length lengths (alpha 1.6, n = 8192), H = 4 heads, d = 128, bf16
storage, seeded synthetic inputs resident in HBM before timing starts.

Throughput is algorithmic causal TFLOP/s: forward 4*d flops per causal
(query, key) pair per head, backward 8*d (four products), i.e.
2*H*d*sum L(L+1) and twice that.  The K timed steps run twice after the
warm-up: first plain, which gives the step time and "value"; then with HIP
events recorded on the launch stream around each kernel (libhstu's profiling
hooks), which give the per-kernel durations (roofline, kernels) and
"profiled_ms_per_step" (the events add small gaps between launches).

Besides the headline step, the same run times (unless --no-extras) one
HSTU layer forward (f1 + SiLU, attention, LayerNorm gate, f2 + residual) and
one layer backward (with its forward recomputed) on
B = 16 Stochastic-Length sequences at N_max = 4096, D = 512, and M-FALCON
scoring of m = 1024 candidates against a 4096-action history (2 layers,
b_m = 256).  These are reported under "extras"; they are not part of "value".

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extras]
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
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
CSRC = os.path.join(ROOT, "hstu_sequential_transducer_amd", "csrc")

# HBM bytes per launch of a kernel on the headline workload, from rocprofv3
# FETCH_SIZE / WRITE_SIZE counter runs scaled by the factor the same counters
# read for a plain device copy of known size.  Valid only for the kernel
# source they were measured on (sha256 over the files listed); otherwise the
# traffic is reported as null.
MEASURED_TRAFFIC = {
    "attn_bwd_bf16_kernel": {"src": "63db4237b98653e2", "bytes": 2274891751},  # read 1464424462 + write 810467289
    "attn_fwd_bf16_kernel": {"src": "a4bec85aa21b7744", "bytes": 450978331},   # read 344233250 + write 106745081
    "dq_gemm_kernel": {"src": "fdc3097f8d6cf2fa", "bytes": 928029683},         # read 892620090 + write 35409593
}


def src_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "attn_bwd_bf16_kernel": ("attn_bwd.hip", "common.h", "kernels.h"),
    "attn_fwd_bf16_kernel": ("attn_fwd.hip", "common.h", "kernels.h"),
    "dq_gemm_kernel": ("dq.hip", "common.h", "kernels.h"),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=80)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--extras-only", action="store_true",
                    help="time only the layer and M-FALCON extras (for a profiler run); prints their JSON")
    ap.add_argument("--cpu-sample-tokens", type=int, default=3072,
                    help="prefix length per sequence for the oracle's timed sample")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (a known-size kernel that "
                         "calibrates HBM byte counters in a profiler run)")
    return ap.parse_args()


def timed(fn, warmup, steps):
    """Run fn warmup times, then time `steps` calls twice: first plain (total
    ms per call from one event pair around all of them, per-call ms from
    events between calls), then again with libhstu's launch-stream events
    around every kernel for the per-kernel durations.  The per-kernel events
    put a small gap between launches (about 4 % of the headline step), so the
    step time comes from the plain pass."""
    import torch
    import hstu_sequential_transducer_amd as hs
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        r = fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
    total = ev[0].elapsed_time(ev[steps]) / steps
    hs.profile_collect()
    hs.profile_enable(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    hs.profile_enable(False)
    kt = hs.profile_collect()
    kernels = {n: {"launches": c, "avg_ms": t / max(c, 1), "total_ms": t} for n, (c, t) in kt.items()}
    return r, total, per, kernels, e0.elapsed_time(e1) / steps


def pct(per):
    return {"median": round(float(np.median(per)), 4), "p10": round(float(np.percentile(per, 10)), 4),
            "p90": round(float(np.percentile(per, 90)), 4)}


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
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(), "cpu_model": cpu_model,
            "kind": "oracle",
            "sample": "fwd+LN gate+bwd of the same 8 sequences cut to their first %d tokens (T=%d, %.1f GFLOP "
                      "algorithmic, %.1f s)" % (prefix, int(lens.sum()), flops / 1e9, dt),
            "seconds": dt}


def _dev_layer(lay, dev):
    import torch
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev).to(torch.bfloat16)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    return dict(w1=bf(lay.w1), b1=f32(lay.b1), w2=bf(lay.w2), b2=f32(lay.b2), rab_p=f32(lay.rab_p),
                rab_t=f32(lay.rab_t), phi1=0)


def bench_layer(args):
    """One HSTU layer forward on B=16 SL(4096, 1.6) sequences, D=512, H=4,
    d=128, bf16."""
    import torch
    import synth
    import hstu_sequential_transducer_amd as hs
    dev = torch.device("cuda:0")
    w = synth.layer_train_4k()
    T, D, H, d = w.total, w.d_model, w.heads, w.d
    lay = _dev_layer(w.layers[0], dev)
    x = torch.from_numpy(w.x).to(dev).to(torch.bfloat16)
    off = torch.from_numpy(w.offsets.astype(np.int32)).to(dev)
    ts = torch.from_numpy(w.ts.astype(np.int64)).to(dev)
    y = torch.empty_like(x)
    nws = hs.binding.workspace_size(hs.binding.OP_LAYER_FWD, hs.binding._jagged(off, ts, w.n_max, T),
                                    hs.binding.Dims(1, H, d, d, w.ln_eps), D, 0)
    wsb = torch.empty(nws, dtype=torch.uint8, device=dev)

    def step():
        return hs.layer_fwd(off, T, ts, x, lay, H, d, w.n_max, eps=w.ln_eps, out=y, workspace=wsb)

    steps = max(10, args.steps // 4)
    _, ms, per, kern, _ = timed(step, args.warmup, steps)
    f_attn = 2.0 * H * d * causal_pairs_sum(w.lengths)
    f_gemm = 2.0 * T * D * 4 * H * d + 2.0 * T * H * d * D
    f1 = 2.0 * T * D * 4 * H * d
    g1, g2 = kern.get("gemm_f1"), kern.get("gemm_f2")
    a = kern.get("attn_fwd_bf16_kernel")
    return {"workload": "layer-fwd B16 SL(4096,1.6) D512 H4 d128 bf16", "tokens": T, "ms": round(ms, 4),
            "step_ms": pct(per), "tokens_per_s": round(T / (ms * 1e-3), 1),
            "f1_tflops": round(f1 / (g1["avg_ms"] * 1e-3) / 1e12, 2) if g1 else None,
            "f2_tflops": round((f_gemm - f1) / (g2["avg_ms"] * 1e-3) / 1e12, 2) if g2 else None,
            "attn_fwd_tflops": round(f_attn / (a["avg_ms"] * 1e-3) / 1e12, 2) if a else None,
            "total_tflops": round((f_gemm + f_attn) / (ms * 1e-3) / 1e12, 2),
            "kernels": {n: {"launches": v["launches"] // steps, "avg_ms": round(v["avg_ms"], 5)} for n, v in kern.items()}}


def bench_layer_bwd(args):
    """One HSTU layer backward (forward recomputed from x inside the call) on
    the same workload as bench_layer, upstream gradient dy ~ N(0, 1)."""
    import torch
    import synth
    import hstu_sequential_transducer_amd as hs
    dev = torch.device("cuda:0")
    w = synth.layer_train_4k()
    T, D, H, d = w.total, w.d_model, w.heads, w.d
    lay = _dev_layer(w.layers[0], dev)
    x = torch.from_numpy(w.x).to(dev).to(torch.bfloat16)
    dy = torch.from_numpy(w.dy).to(dev).to(torch.bfloat16)
    off = torch.from_numpy(w.offsets.astype(np.int32)).to(dev)
    ts = torch.from_numpy(w.ts.astype(np.int64)).to(dev)
    nws = hs.binding.workspace_size(hs.binding.OP_LAYER_BWD, hs.binding._jagged(off, ts, w.n_max, T),
                                    hs.binding.Dims(1, H, d, d, w.ln_eps), D, 0)
    wsb = torch.empty(nws, dtype=torch.uint8, device=dev)

    outs = hs.layer_bwd(off, T, ts, x, lay, dy, H, d, w.n_max, eps=w.ln_eps, workspace=wsb)

    def step():
        return hs.layer_bwd(off, T, ts, x, lay, dy, H, d, w.n_max, eps=w.ln_eps, workspace=wsb, out=outs)

    steps = max(10, args.steps // 4)
    _, ms, per, kern, _ = timed(step, args.warmup, steps)
    pairs2 = causal_pairs_sum(w.lengths)            # 2 x causal pairs per head
    f_attn = 2.0 * H * d * pairs2 * 3               # forward again (4d per pair) + backward (8d per pair)
    f1 = 2.0 * T * D * 4 * H * d                    # f1, dX, dW1: one each
    f2 = 2.0 * T * H * d * D                        # dG, dW2
    total = 3 * f1 + 2 * f2 + f_attn
    w1, w2 = kern.get("gemm_wgrad_w1"), kern.get("gemm_wgrad_w2")
    return {"workload": "layer-bwd B16 SL(4096,1.6) D512 H4 d128 bf16 (forward recomputed)", "tokens": T,
            "ms": round(ms, 4), "step_ms": pct(per), "tokens_per_s": round(T / (ms * 1e-3), 1),
            "total_tflops": round(total / (ms * 1e-3) / 1e12, 2),
            "wgrad_w1_tflops": round(f1 / (w1["avg_ms"] * 1e-3) / 1e12, 2) if w1 else None,
            "wgrad_w2_tflops": round(f2 / (w2["avg_ms"] * 1e-3) / 1e12, 2) if w2 else None,
            "kernels": {n: {"launches": v["launches"] // steps, "avg_ms": round(v["avg_ms"], 5)} for n, v in kern.items()}}


def bench_mfalcon(args):
    """M-FALCON: one user, 4096-action history cached for 2 layers, m = 1024
    candidates in microbatches of b_m = 256."""
    import torch
    import synth
    import hstu_sequential_transducer_amd as hs
    dev = torch.device("cuda:0")
    w = synth.mfalcon_1user()
    T, D, H, d = w.total, w.d_model, w.heads, w.d
    off = torch.from_numpy(w.offsets.astype(np.int32)).to(dev)
    ts = torch.from_numpy(w.ts.astype(np.int64)).to(dev)
    layers = [_dev_layer(l, dev) for l in w.layers]
    h = torch.from_numpy(w.x).to(dev).to(torch.bfloat16)
    kcs, vcs = [], []
    for lay in layers:
        kc = torch.empty((T, H * d), dtype=torch.bfloat16, device=dev)
        vc = torch.empty_like(kc)
        h = hs.layer_fwd(off, T, ts, h, lay, H, d, w.n_max, eps=w.ln_eps, k_cache=kc, v_cache=vc)
        kcs.append(kc)
        vcs.append(vc)
    xc = torch.from_numpy(w.x_cand).to(dev).to(torch.bfloat16)
    M = xc.shape[0]
    co = torch.from_numpy(w.cand_offsets.astype(np.int32)).to(dev)
    cts = torch.from_numpy(w.cand_ts.astype(np.int64)).to(dev)
    nws = hs.binding.workspace_size(hs.binding.OP_MFALCON, hs.binding._jagged(off, ts, w.n_max, T),
                                    hs.binding.Dims(1, H, d, d, w.ln_eps), D, M)
    wsb = torch.empty(nws, dtype=torch.uint8, device=dev)

    def step():
        return hs.mfalcon_score(off, T, ts, layers, kcs, vcs, co, M, cts, xc, w.b_m, H, d, w.n_max,
                                eps=w.ln_eps, workspace=wsb)

    steps = max(10, args.steps // 4)
    _, ms, per, kern, _ = timed(step, args.warmup, steps)
    nl = len(layers)
    f_attn = nl * 4.0 * M * T * d * H
    f_gemm = nl * (2.0 * M * D * 4 * H * d + 2.0 * M * H * d * D)
    a = kern.get("mfalcon_attn_kernel")
    return {"workload": "mfalcon 1 user, history 4096, m=1024, b_m=256, 2 layers, D512 H4 d128 bf16",
            "ms": round(ms, 4), "step_ms": pct(per), "candidates_per_s": round(M / (ms * 1e-3), 1),
            "attn_tflops": round(f_attn / (a["total_ms"] / steps * 1e-3) / 1e12, 2) if a else None,
            "total_tflops": round((f_attn + f_gemm) / (ms * 1e-3) / 1e12, 2),
            "kernels": {n: {"launches": v["launches"] // steps, "avg_ms": round(v["avg_ms"], 5)} for n, v in kern.items()}}


def _dev_attn(w, dev):
    import torch
    T = w.total
    act = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev).to(torch.bfloat16)
    q, k, v = (act(a).reshape(T, w.heads, w.d) for a in (w.q, w.k, w.v))
    return (torch.from_numpy(w.offsets.astype(np.int32)).to(dev), torch.from_numpy(w.ts).to(dev), q, k, v,
            act(w.u), torch.from_numpy(w.rab_p).to(dev), torch.from_numpy(w.rab_t).to(dev))


def _kern(kern, steps):
    return {n: {"launches": v["launches"] // steps, "avg_ms": round(v["avg_ms"], 5)} for n, v in kern.items()}


def bench_fwd_call_8k(args):
    """The forward call alone at the headline shapes (launcher, split-row
    zeroing, attention, LayerNorm gate with O and the statistics saved):
    the spec forward figure, as a fraction of the bf16 MFMA peak."""
    import torch
    import synth
    import hstu_sequential_transducer_amd as hs
    dev = torch.device("cuda:0")
    w = synth.attn_8k(with_grad=False)
    off, ts, q, k, v, u, rp, rt = _dev_attn(w, dev)
    T, F = w.total, w.heads * w.d
    out = torch.empty((T, F), dtype=torch.bfloat16, device=dev)
    osv = torch.empty((T, F), dtype=torch.float32, device=dev)
    lst = torch.empty((T, 2), dtype=torch.float32, device=dev)

    def step():
        return hs.attn_fwd(off, T, ts, q, k, v, rp, rt, w.n_max, u=u, eps=w.ln_eps, out=out, o_save=osv, ln_stats=lst)

    steps = max(20, args.steps)
    _, ms, per, kern, _ = timed(step, args.warmup, steps)
    f = 2.0 * w.heads * w.d * causal_pairs_sum(w.lengths)
    t = f / (ms * 1e-3) / 1e12
    return {"workload": "attn-8k-B8-SL1.6 forward call with the LayerNorm(AV)*U gate", "ms": round(ms, 4),
            "step_ms": pct(per), "tflops": round(t, 2), "pct_mfma_peak": round(100 * t / MFMA_BF16_PEAK_TFLOPS, 2),
            "kernels": _kern(kern, steps)}


def bench_fwd_1k(args):
    """Config 1: bf16 attention forward, B=32, lengths U{64..1024},
    N_max=1024, no gate (O bf16 out)."""
    import torch
    import synth
    import hstu_sequential_transducer_amd as hs
    dev = torch.device("cuda:0")
    w = synth.attn_fwd_1k()
    off, ts, q, k, v, _, rp, rt = _dev_attn(w, dev)
    T, F = w.total, w.heads * w.d
    out = torch.empty((T, F), dtype=torch.bfloat16, device=dev)

    def step():
        return hs.attn_fwd(off, T, ts, q, k, v, rp, rt, w.n_max, out=out)

    steps = max(20, args.steps)
    _, ms, per, kern, _ = timed(step, args.warmup, steps)
    f = 2.0 * w.heads * w.d * causal_pairs_sum(w.lengths)
    t = f / (ms * 1e-3) / 1e12
    return {"workload": "attn-fwd-B32-N1024 (lengths U{64..1024}, no gate)", "tokens": T, "gflop": round(f / 1e9, 2),
            "ms": round(ms, 4), "step_ms": pct(per), "tflops": round(t, 2),
            "pct_mfma_peak": round(100 * t / MFMA_BF16_PEAK_TFLOPS, 2), "kernels": _kern(kern, steps)}


def bench_layer_tiny_f32(args):
    """Config 0: the tiny fp32 layer forward (B=4, lengths {17, 64, 33, 5},
    D=64, H=2, d=32): a latency figure."""
    import torch
    import synth
    import hstu_sequential_transducer_amd as hs
    dev = torch.device("cuda:0")
    w = synth.tiny_layer_f32()
    lay = w.layers[0]
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    dl = dict(w1=f32(lay.w1), b1=f32(lay.b1), w2=f32(lay.w2), b2=f32(lay.b2), rab_p=f32(lay.rab_p),
              rab_t=f32(lay.rab_t), phi1=0)
    x = f32(w.x)
    off = torch.from_numpy(w.offsets.astype(np.int32)).to(dev)
    ts = torch.from_numpy(w.ts).to(dev)
    y = torch.empty_like(x)

    def step():
        return hs.layer_fwd(off, w.total, ts, x, dl, w.heads, w.d, w.n_max, eps=w.ln_eps, out=y)

    steps = max(50, args.steps)
    _, ms, per, kern, _ = timed(step, args.warmup, steps)
    return {"workload": "tiny fp32 layer forward B4 {17,64,33,5} D64 H2 d32", "us": round(ms * 1e3, 2),
            "step_us": {k2: round(v2 * 1e3, 2) for k2, v2 in pct(per).items()}, "kernels": _kern(kern, steps)}


def bench_mfalcon_64(args):
    """Config 4b: M-FALCON over 64 users with SL(4096, 1.6) histories,
    m = 1024 candidates each, 2 layers, b_m = 256."""
    import torch
    import synth
    import hstu_sequential_transducer_amd as hs
    dev = torch.device("cuda:0")
    w = synth.mfalcon_64users()
    T, D, H, d = w.total, w.d_model, w.heads, w.d
    off = torch.from_numpy(w.offsets.astype(np.int32)).to(dev)
    ts = torch.from_numpy(w.ts.astype(np.int64)).to(dev)
    layers = [_dev_layer(l, dev) for l in w.layers]
    h = torch.from_numpy(w.x).to(dev).to(torch.bfloat16)
    kcs, vcs = [], []
    for lay in layers:
        kc = torch.empty((T, H * d), dtype=torch.bfloat16, device=dev)
        vc = torch.empty_like(kc)
        h = hs.layer_fwd(off, T, ts, h, lay, H, d, w.n_max, eps=w.ln_eps, k_cache=kc, v_cache=vc)
        kcs.append(kc)
        vcs.append(vc)
    xc = torch.from_numpy(w.x_cand).to(dev).to(torch.bfloat16)
    M = xc.shape[0]
    co = torch.from_numpy(w.cand_offsets.astype(np.int32)).to(dev)
    cts = torch.from_numpy(w.cand_ts.astype(np.int64)).to(dev)

    def step():
        return hs.mfalcon_score(off, T, ts, layers, kcs, vcs, co, M, cts, xc, w.b_m, H, d, w.n_max, eps=w.ln_eps)

    steps = max(5, args.steps // 4)
    _, ms, per, kern, _ = timed(step, args.warmup, steps)
    nl = len(layers)
    f_attn = nl * 4.0 * (M // len(w.lengths)) * float(w.lengths.sum()) * d * H
    f_gemm = nl * (2.0 * M * D * 4 * H * d + 2.0 * M * H * d * D)
    a = kern.get("mfalcon_attn_kernel")
    return {"workload": "mfalcon 64 users, histories SL(4096,1.6) (T_hist=%d), m=1024 each, b_m=256, 2 layers, "
                        "D512 H4 d128 bf16" % T,
            "ms": round(ms, 4), "step_ms": pct(per), "candidates_per_s": round(M / (ms * 1e-3), 1),
            "attn_tflops": round(f_attn / (a["total_ms"] / steps * 1e-3) / 1e12, 2) if a else None,
            "total_tflops": round((f_attn + f_gemm) / (ms * 1e-3) / 1e12, 2), "kernels": _kern(kern, steps)}


def bench_comparator_8k(args):
    """Pointwise aggregated attention beside its comparator on the same
    kernel skeleton, at the headline shapes, forward only with O out (no
    gate): HSTU with both relative biases, HSTU without them, and causal
    softmax attention (no bias).  Context for the pages' speed-up of HSTU
    over softmax-attention Transformers; the same causal FLOPs in each."""
    import torch
    import synth
    import hstu_sequential_transducer_amd as hs
    dev = torch.device("cuda:0")
    w = synth.attn_8k(with_grad=False)
    off, ts, q, k, v, _, rp, rt = _dev_attn(w, dev)
    T, F = w.total, w.heads * w.d
    out = torch.empty((T, F), dtype=torch.bfloat16, device=dev)
    f = 2.0 * w.heads * w.d * causal_pairs_sum(w.lengths)
    steps = max(20, args.steps // 2)
    res = {"workload": "attn-8k-B8-SL1.6 forward, O out (no gate)", "gflop": round(f / 1e9, 2)}
    runs = {"hstu_rab": lambda: hs.attn_fwd(off, T, ts, q, k, v, rp, rt, w.n_max, out=out),
            "hstu_no_rab": lambda: hs.attn_fwd(off, T, None, q, k, v, None, None, w.n_max, out=out),
            "softmax_no_rab": lambda: hs.softmax_attn_fwd(off, T, q, k, v, w.n_max, out=out)}
    for name, fn in runs.items():
        _, ms, per, kern, _ = timed(fn, args.warmup, steps)
        res[name] = {"ms": round(ms, 4), "tflops": round(f / (ms * 1e-3) / 1e12, 2), "kernels": _kern(kern, steps)}
    res["softmax_over_hstu_rab_time"] = round(res["softmax_no_rab"]["ms"] / res["hstu_rab"]["ms"], 3)
    return res


def bench_sl_sample(args):
    """Stochastic Length sampling of 8 full 8192-action histories (alpha
    1.6) with their 512-wide bf16 rows gathered: the sampled batch's
    construction, as a latency."""
    import torch
    import synth
    import hstu_sequential_transducer_amd as hs
    dev = torch.device("cuda:0")
    L = np.full(8, 8192)
    off_np = synth.offsets_of(L)
    T = int(off_np[-1])
    u, keys = synth.sl_draws(115, L)
    off = torch.from_numpy(off_np).to(dev)
    ts = torch.from_numpy(synth.timestamps(np.random.default_rng(116), L)).to(dev)
    x = torch.randn((T, 512), device=dev).to(torch.bfloat16)
    ud = torch.from_numpy(u).to(dev)
    kd = torch.from_numpy(keys.view(np.int32)).to(dev)

    def step():
        return hs.sl_sample(off, T, ts, 1.6, ud, kd, x)

    steps = max(20, args.steps // 2)
    r, ms, per, kern, _ = timed(step, args.warmup, steps)
    kept = int(r[0][-1].item())
    return {"workload": "SL(alpha 1.6) of 8 x 8192 histories, 512-wide bf16 rows gathered", "kept": kept,
            "ms": round(ms, 4), "step_ms": pct(per), "kernels": _kern(kern, steps)}


def bench_append_64(args):
    """Appending 16 new actions to each of 64 cached users (SL(4096, 1.6)
    histories), one layer: f1, merged caches, attention of the new
    positions, gate, f2."""
    import torch
    import synth
    import hstu_sequential_transducer_amd as hs
    dev = torch.device("cuda:0")
    m = synth.mfalcon_64users()
    w = synth.append_workload("append-64", 96, m.lengths, np.full(64, 16), n_max=4096)
    lay = _dev_layer(w.layers[0], dev)
    T, H, d = w.total, w.heads, w.d
    off = torch.from_numpy(w.offsets.astype(np.int32)).to(dev)
    ts = torch.from_numpy(w.ts).to(dev)
    kc = torch.empty((T, H * d), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    hs.layer_fwd(off, T, ts, torch.from_numpy(w.x).to(dev).to(torch.bfloat16), lay, H, d, w.n_max, k_cache=kc,
                 v_cache=vc)
    aoff = torch.from_numpy(w.add_offsets.astype(np.int32)).to(dev)
    ats = torch.from_numpy(w.add_ts).to(dev)
    xn = torch.from_numpy(w.x_new).to(dev).to(torch.bfloat16)
    Tn = xn.shape[0]
    ko = torch.empty((T + Tn, H * d), dtype=torch.bfloat16, device=dev)
    vo = torch.empty_like(ko)
    y = torch.empty_like(xn)

    def step():
        return hs.layer_append(off, T, ts, aoff, Tn, ats, xn, lay, kc, vc, H, d, w.n_max, out=y, k_out=ko, v_out=vo)

    steps = max(20, args.steps // 2)
    _, ms, per, kern, _ = timed(step, args.warmup, steps)
    return {"workload": "append 16 actions to each of 64 users (T_hist=%d), one layer D512 H4 d128 bf16" % T,
            "ms": round(ms, 4), "step_ms": pct(per), "actions_per_s": round(Tn / (ms * 1e-3), 1),
            "kernels": _kern(kern, steps)}


def all_extras(args):
    return {"fwd_call_8k": bench_fwd_call_8k(args), "fwd_1k": bench_fwd_1k(args),
            "layer_tiny_f32": bench_layer_tiny_f32(args), "layer_fwd": bench_layer(args),
            "layer_bwd": bench_layer_bwd(args), "mfalcon": bench_mfalcon(args), "mfalcon_64users": bench_mfalcon_64(args),
            "comparator_8k": bench_comparator_8k(args), "sl_sample_8k": bench_sl_sample(args),
            "append_64users": bench_append_64(args)}


def hbm_bytes(w, T, H, d):
    """Algorithmic HBM bytes per launch of the bandwidth-bound kernels of the
    headline step (bf16 storage, fp32 O and statistics)."""
    F = H * d
    n_t = (w.lengths + 127) // 128  # key tiles per sequence
    return {"ln_gate_fwd_kernel": T * (4 * F + 2 * F + 2 * F + 8),
            "ln_gate_bwd_kernel": T * (2 * F + 2 * F + 4 * F + 8 + 2 * F + 4 * F),
            "drab_reduce_kernel": int(4 * H * ((n_t * w.lengths).sum() + 64 * n_t.sum()))}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only; --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    import hstu_sequential_transducer_amd as hs

    if args.extras_only:
        print(json.dumps({"extras": all_extras(args)}), flush=True)
        return
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

    g, ms, per, per_kernel, prof_ms = timed(step, args.warmup, args.steps)
    if not all(bool(torch.isfinite(g[n]).all()) for n in ("dq", "dk", "dv", "du", "drab_p", "drab_t")):
        print("bench.py: non-finite gradients", file=sys.stderr)
        sys.exit(1)

    S2 = causal_pairs_sum(w.lengths)
    f_fwd = 2.0 * H * d * S2
    f_bwd = 2.0 * f_fwd
    tflops = (f_fwd + f_bwd) / (ms * 1e-3) / 1e12
    # dominant kernel: the largest share of the timed region.  The backward's
    # four products per pair: dV, dP, dK in attn_bwd, dQ = dS K in dq_gemm.
    dom = max(per_kernel.items(), key=lambda kv: kv[1]["total_ms"])[0]
    kernel_flops = {"attn_bwd_bf16_kernel": 0.75 * f_bwd, "dq_gemm_kernel": 0.25 * f_bwd,
                    "attn_fwd_bf16_kernel": f_fwd}
    dom_flops = kernel_flops.get(dom)
    avg = per_kernel[dom]["avg_ms"]
    roof = None
    if dom_flops is not None:
        ach = dom_flops / (avg * 1e-3) / 1e12
        traffic = None
        mt = MEASURED_TRAFFIC.get(dom)
        if mt and mt["src"] == src_digest(KERNEL_SOURCES[dom]):
            traffic = mt["bytes"]
        roof = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                "traffic_unit": "bytes per launch (HBM read + write)", "avg_ms": round(avg, 4),
                "algorithmic_flops_per_launch": dom_flops, "kernel_src": src_digest(KERNEL_SOURCES[dom])}
    fwd_ms = per_kernel.get("attn_fwd_bf16_kernel", {}).get("avg_ms")
    bwd_ms = per_kernel.get("attn_bwd_bf16_kernel", {}).get("avg_ms")
    dq_ms = per_kernel.get("dq_gemm_kernel", {}).get("avg_ms")
    if bwd_ms and dq_ms:
        bwd_ms += dq_ms
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
        "step_ms": pct(per),
        "profiled_ms_per_step": round(prof_ms, 4),
        "roofline": roof,
        "kernels": {n: {"launches": v2["launches"], "avg_ms": round(v2["avg_ms"], 5)} for n, v2 in per_kernel.items()},
        "attn_fwd_tflops": round(f_fwd / (fwd_ms * 1e-3) / 1e12, 2) if fwd_ms else None,
        "attn_bwd_tflops": round(f_bwd / (bwd_ms * 1e-3) / 1e12, 2) if bwd_ms else None,  # attn_bwd + dq_gemm
        "kernel_tflops": {n: round(f / (per_kernel[n]["avg_ms"] * 1e-3) / 1e12, 2)
                          for n, f in kernel_flops.items() if n in per_kernel},
        # the HBM-bound kernels: algorithmic bytes per launch / average
        # duration (gate forward: O fp32 + U read, G and the stats written;
        # gate backward: dG, U, O, stats read, dU and the dO' hi/lo planes
        # written; the drab reduction: the items' partial sums read)
        "hbm_gbps": {n: round(nb / (per_kernel[n]["avg_ms"] * 1e-3) / 1e9, 1)
                     for n, nb in hbm_bytes(w, T, H, d).items() if n in per_kernel},
    }
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_probe_bytes_each_way"] = n * 4
    if not args.no_extras:
        res["extras"] = all_extras(args)
    if not args.no_cpu_baseline:
        cb = cpu_baseline(w, args.cpu_sample_tokens)
        res["cpu_baseline"] = {k2: (round(v2, 6) if isinstance(v2, float) else v2) for k2, v2 in cb.items()}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
