"""GPU parity of hstu_attn_bwd (through the C ABI) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import BF16_TOL, bf16_bound, host, rel_err, round_bf16, t_act, t_f32, t_i32, t_i64

pytestmark = pytest.mark.gpu

hs = pytest.importorskip("hstu_sequential_transducer_amd")


def gpu_fwd_bwd(w, epilogue=True, use_t=True, use_p=True, eps=None):
    eps = w.ln_eps if eps is None else eps
    T = w.total
    F = w.heads * w.d
    q, k, v = (t_act(a, "bf16").reshape(T, w.heads, w.d) for a in (w.q, w.k, w.v))
    u = t_act(w.u, "bf16") if epilogue else None
    dg = t_act(w.dg, "bf16")
    off, ts = t_i32(w.offsets), t_i64(w.ts) if use_t else None
    rp = t_f32(w.rab_p) if use_p else None
    rt = t_f32(w.rab_t) if use_t else None
    osv = torch.empty((T, F), dtype=torch.float32, device=q.device) if epilogue else None
    lst = torch.empty((T, 2), dtype=torch.float32, device=q.device) if epilogue else None
    if epilogue:
        hs.attn_fwd(off, T, ts, q, k, v, rp, rt, w.n_max, u=u, eps=eps, o_save=osv, ln_stats=lst)
    g = hs.attn_bwd(off, T, ts, q, k, v, rp, rt, w.n_max, dg, u=u, o_save=osv, ln_stats=lst, eps=eps)
    torch.cuda.synchronize()
    return g


def with_grad(seed, lengths, n_max=None, act_std=None):
    L = np.array(lengths)
    w = synth.attention_workload("bwd", seed, L, heads=4, d=128, n_max=n_max or int(max(1, L.max())), epilogue=True,
                                 with_grad=True, act_std=act_std)
    return w


def check_du(got, ref, dg):
    """dU = xhat (.) dG, where xhat = Norm(O) carries the forward's error
    (bf16 P in the AV product: about 1 % of its RMS at the worst element).
    In max|err|/RMS a product's error is that of xhat scaled by the other
    factor's local size, so it is checked on the quantity the kernel
    computes: xhat = dU / dG element by element (dG != 0), within 2e-2 of
    RMS(xhat) plus what rounding dU to bf16 alone does to that ratio.  dU
    itself must then sit within the bound that implies:
    (2e-2 RMS(xhat) max|dG| + max|round(dU) - dU|) / RMS(dU)."""
    dg = np.asarray(dg, np.float64)
    nz = dg != 0
    xh_ref, xh_got = ref[nz] / dg[nz], got[nz] / dg[nz]
    e_x = rel_err(xh_got, xh_ref)
    b_x = BF16_TOL + rel_err(round_bf16(ref)[nz] / dg[nz], xh_ref)
    rms_x = np.sqrt(np.mean(xh_ref ** 2))
    rms_u = np.sqrt(np.mean(ref ** 2))
    b_u = (BF16_TOL * rms_x * np.abs(dg).max() + np.abs(round_bf16(ref) - ref).max()) / rms_u
    e_u = rel_err(got, ref)
    print("du: xhat err", e_x, "bound", b_x, "| du err", e_u, "bound", b_u, "(2e-2 + RNE would be",
          bf16_bound(ref), ")")
    assert e_x <= b_x, ("du/dg", e_x, b_x)
    assert e_u <= b_u, ("du", e_u, b_u)
    return e_u


def check_all(g, ref, names=("dq", "dk", "dv", "du", "drab_p", "drab_t"), dg=None):
    errs = {}
    for n in names:
        if ref.get(n) is None or g.get(n) is None:
            continue
        got = host(g[n]).reshape(ref[n].shape)
        if n == "du":
            errs[n] = check_du(got, ref[n], dg)
            continue
        e = rel_err(got, ref[n])
        errs[n] = e
        bound = BF16_TOL if n.startswith("drab") else bf16_bound(ref[n])
        assert e <= bound, (n, e, bound)
    print("rel errs", errs)
    return errs


@pytest.mark.parametrize("epilogue", [True, False])
def test_bwd_small_ragged(epilogue):
    w = with_grad(21, [1, 127, 128, 129, 300, 64, 33], act_std=0.5)
    g = gpu_fwd_bwd(w, epilogue=epilogue)
    ref = oracle.attn_bwd(w.offsets, w.ts, w.q, w.k, w.v, w.rab_p, w.rab_t, w.n_max, w.u if epilogue else None,
                          w.ln_eps, w.dg)
    check_all(g, ref, dg=w.dg)


def test_bwd_without_bias_terms_and_wide_times():
    w = with_grad(22, [260, 77, 5], act_std=0.5)
    for use_t, use_p in [(False, True), (True, False)]:
        g = gpu_fwd_bwd(w, use_t=use_t, use_p=use_p)
        ref = oracle.attn_bwd(w.offsets, w.ts if use_t else None, w.q, w.k, w.v, w.rab_p if use_p else None,
                              w.rab_t if use_t else None, w.n_max, w.u, w.ln_eps, w.dg)
        names = ("dq", "dk", "dv", "du") + (("drab_p",) if use_p else ()) + (("drab_t",) if use_t else ())
        check_all(g, ref, names, dg=w.dg)
    w.ts = (w.ts - synth.EPOCH) * (1 << 24) + synth.EPOCH
    g = gpu_fwd_bwd(w)
    ref = oracle.attn_bwd(w.offsets, w.ts, w.q, w.k, w.v, w.rab_p, w.rab_t, w.n_max, w.u, w.ln_eps, w.dg)
    check_all(g, ref, dg=w.dg)


@pytest.mark.parametrize("lengths", [[300, 41], [41, 300]])
def test_bwd_clip_beyond_n_max(lengths):
    """Sequences longer than n_max: rab_p clips, and the dS buffer (sized
    from n_max) overflows, so dQ of the sequences that do not fit takes the
    fp32-atomic path ([41, 300]: the first fits, the second does not)."""
    w = with_grad(23, lengths, n_max=100, act_std=0.5)
    g = gpu_fwd_bwd(w)
    ref = oracle.attn_bwd(w.offsets, w.ts, w.q, w.k, w.v, w.rab_p, w.rab_t, w.n_max, w.u, w.ln_eps, w.dg)
    check_all(g, ref, dg=w.dg)


def test_bwd_normalising_regime():
    w = with_grad(24, [200, 90], act_std=1.0)
    g = gpu_fwd_bwd(w, eps=1e-12)
    ref = oracle.attn_bwd(w.offsets, w.ts, w.q, w.k, w.v, w.rab_p, w.rab_t, w.n_max, w.u, 1e-12, w.dg)
    check_all(g, ref, dg=w.dg)


def test_bwd_layer_train_shapes_cap_lengths():
    """B=16 sequences of 777 tokens (the length the SL cap reading gives at
    n=4096, alpha=1.6), N_max=4096, H=4, d=128: full parity of every gradient."""
    w = synth.attention_workload("bwd-777", 3, np.full(16, 777), heads=4, d=128, n_max=4096, epilogue=True,
                                 with_grad=True)
    g = gpu_fwd_bwd(w)
    ref = oracle.attn_bwd(w.offsets, w.ts, w.q, w.k, w.v, w.rab_p, w.rab_t, w.n_max, w.u, w.ln_eps, w.dg)
    check_all(g, ref, dg=w.dg)


@pytest.mark.timeout(1200)
def test_bwd_full_size_8k_every_element():
    """B=8 SL lengths at N_max=8192: the full launch that the benchmark times.
    Every element of dq, dk, dv, du, drab_p and drab_t against one full run
    of the oracle's backward (about 530 GFLOP of fp64 on the host), plus
    identities that hold at any size: sum(drab_p[h]) = sum(drab_t[h]) = sum
    of dS, and sum_i dq_i.q_i = sum_j dk_j.k_j (= sum dS_ij q_i.k_j) per
    head."""
    w = synth.attn_8k(with_grad=True)
    print("case bwd 8k T", w.total, flush=True)
    g = gpu_fwd_bwd(w)
    ref = oracle.attn_bwd(w.offsets, w.ts, w.q, w.k, w.v, w.rab_p, w.rab_t, w.n_max, w.u, w.ln_eps, w.dg)
    errs = check_all(g, ref, dg=w.dg)
    print("8k bwd errors", errs, flush=True)
    drp, drt = host(g["drab_p"]), host(g["drab_t"])
    q, k = w.q.astype(np.float64), w.k.astype(np.float64)
    dqa, dka = host(g["dq"]).reshape(q.shape), host(g["dk"]).reshape(k.shape)
    for h in range(w.heads):
        a, b = drp[h].sum(), drt[h].sum()
        scale = np.abs(drp[h]).sum()
        assert abs(a - b) <= 1e-3 * scale, (h, a, b)
        x = (dqa[:, h] * q[:, h]).sum()
        y = (dka[:, h] * k[:, h]).sum()
        sc = np.abs(dqa[:, h] * q[:, h]).sum()
        assert abs(x - y) <= 2e-2 * sc, (h, x, y)


def test_bwd_deterministic_bitwise():
    """Two backward calls on the same inputs give bit-identical dq, dk, dv,
    du, drab_p and drab_t: the bias gradients are summed in a fixed order
    (per-item partial sums added by sequence, key - query and key tile), not
    with atomics.  B=16 sequences of 777 tokens plus ragged ones."""
    L = np.concatenate([np.full(12, 777), [1, 130, 2000, 64]])
    w = synth.attention_workload("bwd-det", 25, L, heads=4, d=128, n_max=4096, epilogue=True, with_grad=True)
    g1 = gpu_fwd_bwd(w)
    g2 = gpu_fwd_bwd(w)
    for n in ("dq", "dk", "dv", "du", "drab_p", "drab_t"):
        assert torch.equal(g1[n], g2[n]), n


def test_bwd_neighbours_nan():
    """NaN in the other sequences' Q, K, V, U and upstream gradient: the
    gradients of sequence 1 are bit-identical to a clean run (drab tables
    then differ, as they sum over every sequence, so they are not
    compared)."""
    L = [260, 190, 70]
    w = with_grad(26, L, act_std=0.5)
    base = gpu_fwd_bwd(w)
    w2 = with_grad(26, L, act_std=0.5)
    for a in (w2.q, w2.k, w2.v, w2.u, w2.dg):
        a[:260] = np.nan
        a[450:] = np.nan
    g = gpu_fwd_bwd(w2)
    for n in ("dq", "dk", "dv", "du"):
        assert torch.equal(g[n][260:450], base[n][260:450]), n
        assert not torch.isnan(g[n][260:450].float()).any(), n


@pytest.mark.timeout(600)
def test_fwd_bwd_maximum_length():
    """The longest sequence the headline configuration allows, L = N_max =
    8192 (64 key tiles of 128, 128 of 64: the largest split forward items,
    the largest dS plane and every key - query value in [-(N_max - 1), 0]),
    batched with a 37-token and a 1-token sequence: every element of G and of
    the fp32 O, and of dq, dk, dv, du, drab_p and drab_t, against the oracle
    (about 240 GFLOP of fp64 on the host)."""
    w = synth.attention_workload("max-len", 27, np.array([8192, 37, 1]), heads=4, d=128, n_max=8192,
                                 epilogue=True, with_grad=True)
    print("case max length T", w.total, flush=True)
    T, F = w.total, w.heads * w.d
    q, k, v = (t_act(a, "bf16").reshape(T, w.heads, w.d) for a in (w.q, w.k, w.v))
    u = t_act(w.u, "bf16")
    off, ts = t_i32(w.offsets), t_i64(w.ts)
    rp, rt = t_f32(w.rab_p), t_f32(w.rab_t)
    osv = torch.empty((T, F), dtype=torch.float32, device=q.device)
    lst = torch.empty((T, 2), dtype=torch.float32, device=q.device)
    G = hs.attn_fwd(off, T, ts, q, k, v, rp, rt, w.n_max, u=u, eps=w.ln_eps, o_save=osv, ln_stats=lst)
    g = hs.attn_bwd(off, T, ts, q, k, v, rp, rt, w.n_max, t_act(w.dg, "bf16"), u=u, o_save=osv, ln_stats=lst,
                    eps=w.ln_eps)
    torch.cuda.synchronize()
    O = oracle.attn_fwd(w.offsets, w.ts, w.q, w.k, w.v, w.rab_p, w.rab_t, w.n_max)
    Gr, _ = oracle.ln_gate(O, w.u, w.ln_eps)
    eo, eg = rel_err(host(osv), O), rel_err(host(G), Gr)
    print("max length fwd errors O", eo, "G", eg, "bound", bf16_bound(Gr), flush=True)
    assert eo <= BF16_TOL
    assert eg <= bf16_bound(Gr)
    ref = oracle.attn_bwd(w.offsets, w.ts, w.q, w.k, w.v, w.rab_p, w.rab_t, w.n_max, w.u, w.ln_eps, w.dg)
    errs = check_all(g, ref, dg=w.dg)
    print("max length bwd errors", errs, flush=True)


def test_empty_batch():
    """A batch whose every sequence is empty (B = 3, total = 0): the forward
    with and without the gate and the backward return OK with NULL (empty)
    activation views, and the backward's bias gradients, which are
    overwritten, never accumulated, come back as exact zeros."""
    w = synth.attention_workload("empty", 28, np.array([0, 0, 0]), heads=4, d=128, n_max=64, epilogue=True,
                                 with_grad=True)
    assert w.total == 0
    dev = torch.device("cuda:0")
    e = lambda *s: torch.empty(s, dtype=torch.bfloat16, device=dev)
    q, k, v, u, dg = e(0, 4, 128), e(0, 4, 128), e(0, 4, 128), e(0, 512), e(0, 512)
    off, ts = t_i32(w.offsets), t_i64(w.ts)
    rp, rt = t_f32(w.rab_p), t_f32(w.rab_t)
    G = hs.attn_fwd(off, 0, ts, q, k, v, rp, rt, w.n_max, u=u, eps=w.ln_eps)
    O = hs.attn_fwd(off, 0, ts, q, k, v, rp, rt, w.n_max)
    g = hs.attn_bwd(off, 0, ts, q, k, v, rp, rt, w.n_max, dg)
    torch.cuda.synchronize()
    assert G.shape == (0, 512) and O.shape == (0, 512) and g["dq"].shape == (0, 4, 128)
    assert torch.count_nonzero(g["drab_p"]) == 0 and torch.count_nonzero(g["drab_t"]) == 0
