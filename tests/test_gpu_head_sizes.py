"""GPU parity of bf16 attention at head sizes d = 64 and d = 32
(hstu_attn_fwd, hstu_attn_fwd_noalloc, hstu_softmax_attn_fwd and
hstu_attn_bwd through the C ABI) against the fp64 oracle.  The kernels are
the d = 128 ones instantiated for the smaller head: tiles of [rows][d], d/16
MFMA steps for the d contractions, d/32 column blocks for the d-wide
accumulators, and no split of long forward query tiles."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import BF16_TOL, F32_TOL, bf16_bound, host, rel_err, t_act, t_f32, t_i32, t_i64

pytestmark = pytest.mark.gpu

hs = pytest.importorskip("hstu_sequential_transducer_amd")

HEADS = [64, 32]
RAGGED = [1, 127, 128, 129, 300, 64, 33, 0, 5]


def work(seed, lengths, d, H=4, n_max=None, epilogue=False, act_std=0.5):
    L = np.array(lengths)
    return synth.attention_workload("heads", seed, L, heads=H, d=d, n_max=n_max or int(max(1, L.max())),
                                    epilogue=epilogue, act_std=act_std)


def run(w, epi=False, use_t=True, use_p=True, noalloc=False, eps=None):
    T = w.total
    q, k, v = (t_act(a, "bf16").reshape(T, w.heads, w.d) for a in (w.q, w.k, w.v))
    u = t_act(w.u, "bf16") if epi else None
    osv = torch.empty((T, w.heads * w.d), dtype=torch.float32, device=q.device)
    fn = hs.attn_fwd_noalloc if noalloc else hs.attn_fwd
    out = fn(t_i32(w.offsets), T, t_i64(w.ts) if use_t else None, q, k, v, t_f32(w.rab_p) if use_p else None,
             t_f32(w.rab_t) if use_t else None, w.n_max, u=u, eps=w.ln_eps if eps is None else eps, o_save=osv)
    torch.cuda.synchronize()
    return out, osv


def ref(w, epi=False, use_t=True, use_p=True, rows=None):
    O = oracle.attn_fwd(w.offsets, w.ts if use_t else None, w.q, w.k, w.v, w.rab_p if use_p else None,
                        w.rab_t if use_t else None, w.n_max, rows=rows)
    if not epi:
        return O, O
    G, _ = oracle.ln_gate(O, w.u if rows is None else w.u[rows], w.ln_eps)
    return G, O


@pytest.mark.parametrize("d", HEADS)
@pytest.mark.parametrize("epi", [False, True], ids=["plain", "gate"])
def test_fwd_head_size_ragged(d, epi):
    w = work(40 + d, RAGGED, d, epilogue=epi)
    out, osv = run(w, epi=epi)
    G, O = ref(w, epi=epi)
    e, e32 = rel_err(host(out), G), rel_err(host(osv), O)
    print("d", d, "gate" if epi else "plain", "out err", e, "fp32 O err", e32, flush=True)
    assert e32 <= BF16_TOL
    assert e <= bf16_bound(G)


@pytest.mark.parametrize("d", HEADS)
def test_fwd_head_size_bias_terms_and_time_modes(d):
    """Each bias term off in turn, and timestamps spanning beyond 2^32 s (the
    exact 64-bit bucket path)."""
    w = work(50 + d, [200, 31, 96], d)
    for use_t, use_p in [(False, True), (True, False), (False, False)]:
        out, osv = run(w, use_t=use_t, use_p=use_p)
        G, _ = ref(w, use_t=use_t, use_p=use_p)
        assert rel_err(host(osv), G) <= BF16_TOL, (use_t, use_p)
        assert rel_err(host(out), G) <= bf16_bound(G), (use_t, use_p)
    w.ts = (w.ts - synth.EPOCH) * (1 << 24) + synth.EPOCH
    out, osv = run(w)
    G, _ = ref(w)
    assert rel_err(host(osv), G) <= BF16_TOL
    assert rel_err(host(out), G) <= bf16_bound(G)


@pytest.mark.parametrize("d", HEADS)
def test_fwd_head_size_long_gate_sampled_rows(d):
    """Long sequences through the gate path (whose d = 128 kernel splits long
    query tiles; these sizes never split), rows sampled across every tile
    position, positions clipped by n_max below the longest length."""
    w = work(60 + d, [2100, 1, 700, 1500], d, H=8, n_max=1800, epilogue=True, act_std=1.0)
    out, osv = run(w, epi=True, eps=1e-12)
    rng = np.random.default_rng(d)
    rows = np.unique(np.concatenate([rng.choice(w.total, 300, replace=False), [0, w.total - 1, 2099, 2100, 2101]]))
    O = oracle.attn_fwd(w.offsets, w.ts, w.q, w.k, w.v, w.rab_p, w.rab_t, w.n_max, rows=rows)
    G, _ = oracle.ln_gate(O, w.u[rows], 1e-12)
    assert rel_err(host(osv)[rows], O) <= BF16_TOL
    assert rel_err(host(out)[rows], G) <= bf16_bound(G)


@pytest.mark.parametrize("d", HEADS)
def test_noalloc_head_size_matches_workspace_path(d):
    """The allocation-free entry point at the smaller head: bit-identical to
    hstu_attn_fwd on two calls in a row, the second with a smaller batch."""
    for seed, lengths in ((70, [300, 129, 7]), (71, [65, 2])):
        w = work(seed + d, lengths, d, epilogue=True)
        a, a32 = run(w, epi=True)
        b, b32 = run(w, epi=True, noalloc=True)
        assert torch.equal(a, b) and torch.equal(a32, b32)


@pytest.mark.parametrize("d", HEADS)
def test_softmax_head_size(d):
    w = work(80 + d, [1, 127, 128, 129, 300, 0, 700], d, act_std=1.0)
    T = w.total
    q, k, v = (t_act(a, "bf16").reshape(T, w.heads, w.d) for a in (w.q, w.k, w.v))
    lse = torch.empty((T, w.heads), dtype=torch.float32, device=q.device)
    out = hs.softmax_attn_fwd(t_i32(w.offsets), T, q, k, v, w.n_max, lse=lse)
    torch.cuda.synchronize()
    O, lref = oracle.softmax_attn_fwd(w.offsets, w.q, w.k, w.v, want_lse=True)
    e, el = rel_err(host(out), O), rel_err(host(lse), lref)
    print("softmax d", d, "O err", e, "lse err", el, flush=True)
    assert e <= bf16_bound(O)
    assert el <= F32_TOL


# ---------------------------------------------------------------- backward

def bwd_work(seed, lengths, d, n_max=None, act_std=0.5, H=4):
    L = np.array(lengths)
    return synth.attention_workload("heads-bwd", seed, L, heads=H, d=d, n_max=n_max or int(max(1, L.max())),
                                    epilogue=True, with_grad=True, act_std=act_std)


def gpu_fwd_bwd(w, epi=True, use_t=True, use_p=True):
    T, F = w.total, w.heads * w.d
    q, k, v = (t_act(a, "bf16").reshape(T, w.heads, w.d) for a in (w.q, w.k, w.v))
    u = t_act(w.u, "bf16") if epi else None
    dg = t_act(w.dg, "bf16")
    off, ts = t_i32(w.offsets), t_i64(w.ts) if use_t else None
    rp = t_f32(w.rab_p) if use_p else None
    rt = t_f32(w.rab_t) if use_t else None
    osv = torch.empty((T, F), dtype=torch.float32, device=q.device) if epi else None
    lst = torch.empty((T, 2), dtype=torch.float32, device=q.device) if epi else None
    if epi:
        hs.attn_fwd(off, T, ts, q, k, v, rp, rt, w.n_max, u=u, eps=w.ln_eps, o_save=osv, ln_stats=lst)
    g = hs.attn_bwd(off, T, ts, q, k, v, rp, rt, w.n_max, dg, u=u, o_save=osv, ln_stats=lst, eps=w.ln_eps)
    torch.cuda.synchronize()
    return g


def check_bwd(g, ref, w, names=("dq", "dk", "dv", "du", "drab_p", "drab_t")):
    from test_gpu_attn_bwd import check_all
    return check_all(g, ref, names, dg=w.dg)


@pytest.mark.parametrize("d", HEADS)
@pytest.mark.parametrize("epi", [True, False], ids=["gate", "plain"])
def test_bwd_head_size_ragged(d, epi):
    """Every gradient at d = 64 and d = 32 on a ragged batch: partial query
    blocks, one-token and empty sequences, several key tiles."""
    w = bwd_work(100 + d, RAGGED, d)
    g = gpu_fwd_bwd(w, epi=epi)
    ref = oracle.attn_bwd(w.offsets, w.ts, w.q, w.k, w.v, w.rab_p, w.rab_t, w.n_max, w.u if epi else None,
                          w.ln_eps, w.dg)
    print("bwd d", d, "gate" if epi else "plain", flush=True)
    check_bwd(g, ref, w)


@pytest.mark.parametrize("d", HEADS)
def test_bwd_head_size_bias_modes_and_wide_times(d):
    w = bwd_work(110 + d, [260, 77, 5], d)
    for use_t, use_p in [(False, True), (True, False)]:
        g = gpu_fwd_bwd(w, use_t=use_t, use_p=use_p)
        ref = oracle.attn_bwd(w.offsets, w.ts if use_t else None, w.q, w.k, w.v, w.rab_p if use_p else None,
                              w.rab_t if use_t else None, w.n_max, w.u, w.ln_eps, w.dg)
        names = ("dq", "dk", "dv", "du") + (("drab_p",) if use_p else ()) + (("drab_t",) if use_t else ())
        check_bwd(g, ref, w, names)
    w.ts = (w.ts - synth.EPOCH) * (1 << 24) + synth.EPOCH
    g = gpu_fwd_bwd(w)
    ref = oracle.attn_bwd(w.offsets, w.ts, w.q, w.k, w.v, w.rab_p, w.rab_t, w.n_max, w.u, w.ln_eps, w.dg)
    check_bwd(g, ref, w)


@pytest.mark.parametrize("d", HEADS)
def test_bwd_head_size_beyond_n_max_and_deterministic(d):
    """Sequences longer than n_max (clipped positions; the second one's dS
    plane does not fit the buffer sized from n_max, so its dQ goes through
    the fp32-atomic path), then a longer batch twice: every output
    bit-identical."""
    w = bwd_work(120 + d, [41, 300], d, n_max=100)
    g = gpu_fwd_bwd(w)
    ref = oracle.attn_bwd(w.offsets, w.ts, w.q, w.k, w.v, w.rab_p, w.rab_t, w.n_max, w.u, w.ln_eps, w.dg)
    check_bwd(g, ref, w)
    w = bwd_work(130 + d, [777, 1, 1500, 64, 333], d, n_max=2048, H=8)
    g1 = gpu_fwd_bwd(w)
    g2 = gpu_fwd_bwd(w)
    for n in ("dq", "dk", "dv", "du", "drab_p", "drab_t"):
        assert torch.equal(g1[n], g2[n]), n
    ref = oracle.attn_bwd(w.offsets, w.ts, w.q, w.k, w.v, w.rab_p, w.rab_t, w.n_max, w.u, w.ln_eps, w.dg)
    check_bwd(g1, ref, w)


def test_head_size_128_only_entry_points_refuse_smaller_heads():
    """The layer entry points keep d = 128: a d = 64 layer forward returns
    HSTU_ERR_UNSUPPORTED before any device work."""
    H, d, D = 4, 64, 256
    L = np.array([40, 9])
    T = int(L.sum())
    dev_ = torch.device("cuda:0")
    x = torch.zeros((T, D), dtype=torch.bfloat16, device=dev_)
    lay = {"w1": torch.zeros((4 * H * d, D), dtype=torch.bfloat16, device=dev_), "b1": None,
           "w2": torch.zeros((D, H * d), dtype=torch.bfloat16, device=dev_), "b2": None,
           "rab_p": None, "rab_t": None, "phi1": hs.HSTU_ACT_SILU}
    with pytest.raises(hs.HstuError, match="d = 128"):
        hs.layer_fwd(t_i32(synth.offsets_of(L)), T, None, x, lay, H, d, 64)
