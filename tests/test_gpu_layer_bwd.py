"""GPU parity of hstu_layer_bwd (through the C ABI) against the fp64 oracle's
layer backward (chain rule through f2 and the residual, Norm (.) U, Eq. 2,
phi1 and f1): dx, dw1, db1, dw2, db2, drab_p, drab_t."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import BF16_TOL, bf16_bound, host, rel_err, t_act, t_f32, t_i32, t_i64

pytestmark = pytest.mark.gpu

hs = pytest.importorskip("hstu_sequential_transducer_amd")


def strong(w, seed):
    """Weights of std 1/sqrt(fan_in), biases and tables of std 0.1/0.5 (bf16
    weights), so every stage of the layer is in its non-linear range."""
    rng = np.random.default_rng(seed)
    lay = w.layers[0]
    D, HD = w.d_model, w.heads * w.d
    lay.w1 = synth.round_bf16(rng.standard_normal(lay.w1.shape).astype(np.float32) / math.sqrt(D))
    lay.w2 = synth.round_bf16(rng.standard_normal(lay.w2.shape).astype(np.float32) / math.sqrt(HD))
    lay.b1 = (rng.standard_normal(4 * HD) * 0.1).astype(np.float32)
    lay.b2 = (rng.standard_normal(D) * 0.1).astype(np.float32)
    lay.rab_p = (rng.standard_normal(lay.rab_p.shape) * 0.5).astype(np.float32)
    lay.rab_t = (rng.standard_normal(lay.rab_t.shape) * 0.5).astype(np.float32)
    return lay


def run(w, lay, phi1, with_ts=True, want_bias_grads=True):
    T = w.total
    dl = dict(w1=t_act(lay.w1, "bf16"), b1=t_f32(lay.b1), w2=t_act(lay.w2, "bf16"), b2=t_f32(lay.b2),
              rab_p=t_f32(lay.rab_p), rab_t=t_f32(lay.rab_t), phi1=phi1)
    ts = t_i64(w.ts) if with_ts else None
    g = hs.layer_bwd(t_i32(w.offsets), T, ts, t_act(w.x, "bf16"), dl, t_act(w.dy, "bf16"), w.heads, w.d, w.n_max,
                     want_bias_grads=want_bias_grads)
    torch.cuda.synchronize()
    return g


def storage_error(w, lay, phi1, ref, return_emulation=False):
    """The error that bf16 storage of the layer's intermediate activations
    alone causes, per output, as max|err|/RMS against the fp64 oracle: the
    chain rule evaluated in fp64 from the oracle's own pieces (attention
    forward, gate, attention backward), with every tensor the library keeps
    in bf16 rounded to bf16 where it is stored -- phi1(Z) (U, V, Q, K), Z
    for phi1', G, dG, the gradient at phi1(Z) and dZ.  The GPU result may
    differ from the oracle by this much before its own arithmetic counts."""
    rb = lambda a: synth.round_bf16(np.asarray(a, np.float32)).astype(np.float64)
    T, D, H, d = w.total, w.d_model, w.heads, w.d
    HD = H * d
    X, dY = w.x.astype(np.float64), w.dy.astype(np.float64)
    W1, W2 = lay.w1.astype(np.float64), lay.w2.astype(np.float64)
    Z = X @ W1.T + lay.b1
    if phi1 == 1:
        A, dphi = np.maximum(Z, 0.0), (rb(Z) > 0).astype(np.float64)
    else:
        sg = 1.0 / (1.0 + np.exp(-Z))
        A = Z * sg
        zr = rb(Z)
        sr = 1.0 / (1.0 + np.exp(-zr))
        dphi = sr * (1.0 + zr * (1.0 - sr))
    A = rb(A)
    U, V, Q, K = (A[:, i * HD:(i + 1) * HD] for i in range(4))
    three = lambda M: M.reshape(T, H, d)
    O = oracle.attn_fwd(w.offsets, w.ts, three(Q), three(K), three(V), lay.rab_p, lay.rab_t, w.n_max).reshape(T, HD)
    G = rb(oracle.ln_gate(O, U, 1e-5)[0])
    dG = rb(dY @ W2)
    g = oracle.attn_bwd(w.offsets, w.ts, three(Q), three(K), three(V), lay.rab_p, lay.rab_t, w.n_max, U, 1e-5, dG)
    dA = rb(np.concatenate([g["du"], g["dv"].reshape(T, HD), g["dq"].reshape(T, HD), g["dk"].reshape(T, HD)], 1))
    dZ = rb(dA * dphi)
    emu = dict(dx=dY + dZ @ W1, dw1=dZ.T @ X, db1=dZ.sum(0), dw2=dY.T @ G, db2=dY.sum(0), drab_p=g["drab_p"],
               drab_t=g["drab_t"])
    errs = {k: rel_err(emu[k], ref[k]) for k in ref if ref[k] is not None}
    return (errs, emu) if return_emulation else errs


def check(g, ref, names, tag, store_err):
    """max|err|/RMS <= 2e-2 + the storage error of that output (plus, for dx,
    its own bf16 rounding: 2^-8 of its peak over its RMS)."""
    bad = []
    for name in names:
        got, exp = host(g[name]), ref[name]
        bound = (bf16_bound(exp) if name == "dx" else BF16_TOL) + store_err[name]
        e = rel_err(got, exp)
        print(tag, name, "err", e, "storage err", store_err[name], "bound", bound, flush=True)
        if e > bound:
            bad.append((name, e, bound))
    assert not bad, bad


ALL = ["dx", "dw1", "db1", "dw2", "db2", "drab_p", "drab_t"]


@pytest.mark.parametrize("phi1", [0, 1])
def test_layer_bwd_small(phi1):
    """D=64, H=1, d=128, lengths {70, 130, 3, 64, 1} (T=268: partial token
    steps, a one-token sequence, several row tiles), N_max=192."""
    L = np.array([70, 130, 3, 64, 1])
    w = synth.layer_workload("layer-bwd-small", 51 + phi1, L, d_model=64, heads=1, d=128, n_max=192, dtype="bf16",
                             with_grad=True)
    lay = strong(w, 61 + phi1)
    print("case layer_bwd_small phi1", phi1, "T", w.total, flush=True)
    g = run(w, lay, phi1)
    ref = oracle.layer_bwd(w.offsets, w.ts, w.x, lay, w.dy, w.heads, w.d, w.n_max, phi1=phi1)
    check(g, ref, ALL, "small phi1=%d" % phi1, storage_error(w, lay, phi1, ref))


def test_layer_bwd_multihead():
    """D=512, H=4, d=128, lengths {100, 300, 1, 64, 129} (T=594), N_max=512:
    the layer's real widths (f1 2048 wide) on a ragged batch."""
    L = np.array([100, 300, 1, 64, 129])
    w = synth.layer_workload("layer-bwd-mh", 53, L, d_model=512, heads=4, d=128, n_max=512, dtype="bf16",
                             with_grad=True)
    lay = strong(w, 63)
    print("case layer_bwd_multihead T", w.total, flush=True)
    g = run(w, lay, 0)
    ref = oracle.layer_bwd(w.offsets, w.ts, w.x, lay, w.dy, w.heads, w.d, w.n_max)
    check(g, ref, ALL, "multihead", storage_error(w, lay, 0, ref))


def test_layer_bwd_no_timestamps_no_bias_grads():
    """No timestamps (no rab_t term, no drab_t), db1 and db2 not requested,
    and an empty sequence inside the batch."""
    L = np.array([33, 0, 97, 128])
    w = synth.layer_workload("layer-bwd-nots", 55, L, d_model=128, heads=2, d=128, n_max=128, dtype="bf16",
                             with_grad=True)
    lay = strong(w, 65)
    print("case layer_bwd_no_ts T", w.total, flush=True)
    g = run(w, lay, 0, with_ts=False, want_bias_grads=False)
    assert g["db1"] is None and g["db2"] is None and g["drab_t"] is None
    lay_nt = synth.Layer(lay.w1, lay.b1, lay.w2, lay.b2, lay.rab_p, None)
    ref = oracle.layer_bwd(w.offsets, w.ts, w.x, lay_nt, w.dy, w.heads, w.d, w.n_max)
    check(g, ref, ["dx", "dw1", "dw2", "drab_p"], "no-ts", storage_error(w, lay_nt, 0, ref))


def test_layer_bwd_full_size_properties():
    """The layer training workload (B=16, SL lengths up to 4096, D=512, H=4,
    d=128): db2 equals the column sums of dy (exact up to fp32 summation of
    bf16 values), two calls give bit-identical dx and weight and bias
    gradients (the split sums are added in a fixed order; the rab table
    gradients are accumulated with atomics and may differ in rounding), and
    every output is finite."""
    w = synth.layer_train_4k()
    lay = strong(w, 67)
    print("case layer_bwd_full T", w.total, flush=True)
    g1 = run(w, lay, 0)
    g2 = run(w, lay, 0)
    for name in ALL:
        assert torch.isfinite(g1[name].float()).all(), name
        if not name.startswith("drab"):
            assert torch.equal(g1[name], g2[name]), name
    cs = w.dy.astype(np.float64).sum(axis=0)
    e = np.abs(host(g1["db2"]) - cs).max() / np.sqrt(np.mean(cs ** 2))
    print("full db2 err", e, flush=True)
    assert e <= 1e-5


def subset(w, seqs):
    """The listed sequences of a layer workload as a batch of their own (a
    sequence's gradients at its own rows depend on that sequence alone)."""
    seqs = np.asarray(seqs)
    rows = np.concatenate([np.arange(w.offsets[b], w.offsets[b + 1]) for b in seqs])
    L = w.lengths[seqs]
    sub = synth.Workload(name=w.name + "-subset", dtype=w.dtype, heads=w.heads, d=w.d, n_max=w.n_max, lengths=L,
                         offsets=synth.offsets_of(L), ts=w.ts[rows], rab_p=w.rab_p, rab_t=w.rab_t,
                         d_model=w.d_model, layers=w.layers, x=w.x[rows], dy=w.dy[rows])
    return sub, rows


@pytest.mark.timeout(900)
def test_layer_bwd_4k_own_draws_subset():
    """The layer training workload with its own draws (B=16, SL lengths up to
    4096, D=512, H=4, d=128, weights and tables ~ N(0, 0.02)).  The full
    launch's dx on three sequences (the two shortest and the longest)
    against the oracle's layer backward run on those three alone; then the
    backward of that three-sequence batch on the GPU against the same oracle
    run, every output (the weight and table gradients sum over the batch's
    tokens).  Bound: 2e-2 + the error that bf16 storage of the layer's
    intermediates alone causes (computed from the oracle's own pieces); the
    GPU must also sit within 2e-2 of that bf16-storage emulation itself."""
    w = synth.layer_train_4k()
    lay = w.layers[0]
    seqs = np.sort(np.argsort(w.lengths, kind="stable")[[0, 1, -1]])
    sub, rows = subset(w, seqs)
    print("case layer_bwd_4k_own_draws: full T", w.total, "subset", seqs.tolist(), "lengths", sub.lengths.tolist(),
          flush=True)
    g_full = run(w, lay, 0)
    ref = oracle.layer_bwd(sub.offsets, sub.ts, sub.x, lay, sub.dy, sub.heads, sub.d, sub.n_max)
    se, emu = storage_error(sub, lay, 0, ref, return_emulation=True)
    e = rel_err(host(g_full["dx"])[rows], ref["dx"])
    print("full launch dx on the subset: err", e, "storage err", se["dx"], flush=True)
    assert e <= bf16_bound(ref["dx"]) + se["dx"]
    g = run(sub, lay, 0)
    check(g, ref, ALL, "4k-subset", se)
    for name in ALL:
        got = host(g[name])
        em = np.asarray(emu[name], np.float64).reshape(got.shape)
        e2 = rel_err(got, em)
        bound = bf16_bound(em) if name == "dx" else BF16_TOL
        print("4k-subset", name, "err vs bf16-storage emulation", e2, "bound", bound, flush=True)
        assert e2 <= bound, (name, e2, bound)
