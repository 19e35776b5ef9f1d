"""GPU parity of hstu_attn_bwd (through the C ABI) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import BF16_TOL, bf16_bound, host, rel_err, sample_rows, t_act, t_f32, t_i32, t_i64

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


def check_all(g, ref, names=("dq", "dk", "dv", "du", "drab_p", "drab_t")):
    errs = {}
    for n in names:
        if ref.get(n) is None or g.get(n) is None:
            continue
        got = host(g[n]).reshape(ref[n].shape)
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
    check_all(g, ref)


def test_bwd_without_bias_terms_and_wide_times():
    w = with_grad(22, [260, 77, 5], act_std=0.5)
    for use_t, use_p in [(False, True), (True, False)]:
        g = gpu_fwd_bwd(w, use_t=use_t, use_p=use_p)
        ref = oracle.attn_bwd(w.offsets, w.ts if use_t else None, w.q, w.k, w.v, w.rab_p if use_p else None,
                              w.rab_t if use_t else None, w.n_max, w.u, w.ln_eps, w.dg)
        names = ("dq", "dk", "dv", "du") + (("drab_p",) if use_p else ()) + (("drab_t",) if use_t else ())
        check_all(g, ref, names)
    w.ts = (w.ts - synth.EPOCH) * (1 << 24) + synth.EPOCH
    g = gpu_fwd_bwd(w)
    ref = oracle.attn_bwd(w.offsets, w.ts, w.q, w.k, w.v, w.rab_p, w.rab_t, w.n_max, w.u, w.ln_eps, w.dg)
    check_all(g, ref)


@pytest.mark.parametrize("lengths", [[300, 41], [41, 300]])
def test_bwd_clip_beyond_n_max(lengths):
    """Sequences longer than n_max: rab_p clips, and the dS buffer (sized
    from n_max) overflows, so dQ of the sequences that do not fit takes the
    fp32-atomic path ([41, 300]: the first fits, the second does not)."""
    w = with_grad(23, lengths, n_max=100, act_std=0.5)
    g = gpu_fwd_bwd(w)
    ref = oracle.attn_bwd(w.offsets, w.ts, w.q, w.k, w.v, w.rab_p, w.rab_t, w.n_max, w.u, w.ln_eps, w.dg)
    check_all(g, ref)


def test_bwd_normalising_regime():
    w = with_grad(24, [200, 90], act_std=1.0)
    g = gpu_fwd_bwd(w, eps=1e-12)
    ref = oracle.attn_bwd(w.offsets, w.ts, w.q, w.k, w.v, w.rab_p, w.rab_t, w.n_max, w.u, 1e-12, w.dg)
    check_all(g, ref)


def test_bwd_layer_train_shapes_cap_lengths():
    """B=16 sequences of 777 tokens (the length the SL cap reading gives at
    n=4096, alpha=1.6), N_max=4096, H=4, d=128: full parity of every gradient."""
    w = synth.attention_workload("bwd-777", 3, np.full(16, 777), heads=4, d=128, n_max=4096, epilogue=True,
                                 with_grad=True)
    g = gpu_fwd_bwd(w)
    ref = oracle.attn_bwd(w.offsets, w.ts, w.q, w.k, w.v, w.rab_p, w.rab_t, w.n_max, w.u, w.ln_eps, w.dg)
    check_all(g, ref)


def test_bwd_full_size_8k_sampled_and_invariants():
    """B=8 SL lengths at N_max=8192: the full launch.  dq and du on sampled
    rows against the oracle; identities that hold at any size for the rest:
    sum(drab_p[h]) = sum(drab_t[h]) = sum of dS, and
    sum_i dq_i.q_i = sum_j dk_j.k_j (= sum dS_ij q_i.k_j) per head."""
    w = synth.attn_8k(with_grad=True)
    g = gpu_fwd_bwd(w)
    rows = sample_rows(w.offsets, 24, np.random.default_rng(3))
    dq_ref = oracle.attn_bwd_dq_rows(w.offsets, w.ts, w.q, w.k, w.v, w.rab_p, w.rab_t, w.n_max, w.u, w.ln_eps, w.dg,
                                     rows)
    dq = host(g["dq"])[rows]
    e = rel_err(dq, dq_ref)
    assert e <= bf16_bound(dq_ref), e
    O = oracle.attn_fwd(w.offsets, w.ts, w.q, w.k, w.v, w.rab_p, w.rab_t, w.n_max, rows=rows)
    xh, _ = oracle.ln_gate(O, np.ones_like(O), w.ln_eps)
    du_ref = xh * w.dg[rows]
    e2 = rel_err(host(g["du"])[rows], du_ref)
    assert e2 <= bf16_bound(du_ref), e2
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
    print("8k bwd dq err", e, "du err", e2)
