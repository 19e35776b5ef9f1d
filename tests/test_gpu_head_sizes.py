"""GPU parity of the bf16 attention forwards at head sizes d = 64 and d = 32
(hstu_attn_fwd, hstu_attn_fwd_noalloc, hstu_softmax_attn_fwd through the C
ABI) against the fp64 oracle.  The kernels are the d = 128 ones instantiated
for the smaller head: K/V tiles of [64][d], d/16 MFMA steps for S, d/32
column blocks for O, and no split of long query tiles."""
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


def test_head_size_128_only_entry_points_refuse_smaller_heads():
    """The backward keeps d = 128: a d = 64 call returns
    HSTU_ERR_UNSUPPORTED before any device work."""
    w = work(90, [40, 9], 64)
    T = w.total
    q, k, v = (t_act(a, "bf16").reshape(T, w.heads, w.d) for a in (w.q, w.k, w.v))
    dout = torch.zeros((T, w.heads * w.d), dtype=torch.bfloat16, device=q.device)
    with pytest.raises(hs.HstuError, match="d = 128"):
        hs.attn_bwd(t_i32(w.offsets), T, t_i64(w.ts), q, k, v, t_f32(w.rab_p), t_f32(w.rab_t), w.n_max, dout)
