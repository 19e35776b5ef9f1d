"""GPU parity of hstu_attn_fwd (through the C ABI) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import BF16_TOL, F32_TOL, bf16_bound, host, rel_err, sample_rows, t_act, t_f32, t_i32, t_i64

pytestmark = pytest.mark.gpu

hs = pytest.importorskip("hstu_sequential_transducer_amd")


def run_fwd(w, epilogue=None, eps=None, o_save=False, stats=False, use_t=True, use_p=True):
    epi = w.epilogue if epilogue is None else epilogue
    eps = w.ln_eps if eps is None else eps
    T = w.total
    q, k, v = (t_act(a, w.dtype) for a in (w.q, w.k, w.v))
    u = t_act(w.u, w.dtype) if epi else None
    osv = torch.empty((T, w.heads * w.d), dtype=torch.float32, device=q.device) if o_save else None
    lst = torch.empty((T, 2), dtype=torch.float32, device=q.device) if stats else None
    out = hs.attn_fwd(t_i32(w.offsets), T, t_i64(w.ts) if use_t else None, q, k, v,
                      t_f32(w.rab_p) if use_p else None, t_f32(w.rab_t) if use_t else None, w.n_max, u=u, eps=eps,
                      o_save=osv, ln_stats=lst)
    torch.cuda.synchronize()
    return out, osv, lst


def ref_fwd(w, rows=None, epilogue=None, eps=None, use_t=True, use_p=True):
    epi = w.epilogue if epilogue is None else epilogue
    eps = w.ln_eps if eps is None else eps
    O = oracle.attn_fwd(w.offsets, w.ts if use_t else None, w.q, w.k, w.v, w.rab_p if use_p else None,
                        w.rab_t if use_t else None, w.n_max, rows=rows)
    if not epi:
        return O, O
    U = w.u if rows is None else w.u[rows]
    G, _ = oracle.ln_gate(O, U, eps)
    return G, O


def small(seed, lengths, H=4, n_max=None, epilogue=False, act_std=None):
    L = np.array(lengths)
    return synth.attention_workload("small", seed, L, heads=H, d=128, n_max=n_max or int(max(1, L.max())),
                                    epilogue=epilogue, act_std=act_std)


CASES = [
    ("ragged", [1, 127, 128, 129, 300, 64, 33]),
    ("single-long", [700]),
    ("tiles-exact", [256, 128, 384]),
    ("with-empty", [0, 5, 0, 200]),
]


@pytest.mark.parametrize("name,lengths", CASES, ids=[c[0] for c in CASES])
def test_fwd_no_epilogue_small(name, lengths):
    w = small(11, lengths, act_std=0.5)
    out, osv, _ = run_fwd(w, o_save=True)
    ref, _ = ref_fwd(w)
    err = rel_err(host(out), ref)
    err32 = rel_err(host(osv), ref)
    print(name, "rel err bf16 out", err, "fp32 O", err32)
    assert err32 <= BF16_TOL
    assert err <= bf16_bound(ref)


@pytest.mark.parametrize("name,lengths", CASES[:2], ids=[c[0] for c in CASES[:2]])
def test_fwd_epilogue_small(name, lengths):
    w = small(12, lengths, epilogue=True, act_std=0.5)
    out, osv, lst = run_fwd(w, o_save=True, stats=True)
    G, O = ref_fwd(w)
    assert rel_err(host(out), G) <= bf16_bound(G)
    assert rel_err(host(osv), O) <= BF16_TOL
    _, st = oracle.ln_gate(O, w.u, w.ln_eps)
    assert rel_err(host(lst)[:, 0], st[:, 0]) <= BF16_TOL
    assert rel_err(host(lst)[:, 1], st[:, 1]) <= BF16_TOL


def test_fwd_epilogue_normalising_regime():
    """eps far below the row variance, so a wrong variance would show."""
    w = small(13, [300, 77], epilogue=True, act_std=1.0)
    out, _, _ = run_fwd(w, eps=1e-12)
    G, _ = ref_fwd(w, eps=1e-12)
    assert rel_err(host(out), G) <= bf16_bound(G)


def test_fwd_without_bias_terms():
    w = small(14, [200, 31])
    for use_t, use_p in [(False, True), (True, False), (False, False)]:
        out, osv, _ = run_fwd(w, use_t=use_t, use_p=use_p, o_save=True)
        ref, _ = ref_fwd(w, use_t=use_t, use_p=use_p)
        assert rel_err(host(osv), ref) <= BF16_TOL, (use_t, use_p)
        assert rel_err(host(out), ref) <= bf16_bound(ref), (use_t, use_p)


def test_fwd_wide_time_span_uses_exact_64bit_buckets():
    w = small(15, [150, 90])
    w.ts = (w.ts - synth.EPOCH) * (1 << 24) + synth.EPOCH   # spans beyond 2^32 s
    out, osv, _ = run_fwd(w, o_save=True)
    ref, _ = ref_fwd(w)
    assert rel_err(host(osv), ref) <= BF16_TOL
    assert rel_err(host(out), ref) <= bf16_bound(ref)


def test_fwd_sequences_longer_than_n_max_clip_positions():
    w = small(16, [300, 40], n_max=100)
    out, osv, _ = run_fwd(w, o_save=True)
    ref, _ = ref_fwd(w)
    assert rel_err(host(osv), ref) <= BF16_TOL
    assert rel_err(host(out), ref) <= bf16_bound(ref)


def run_fwd_padded(w, tail_rows=64, fill=float("nan")):
    """run_fwd with Q, K, V (and the output) as views of buffers that hold
    `tail_rows` extra rows of `fill` past the last token, so a read beyond T
    would show in the result."""
    T, F = w.total, w.heads * w.d
    dev_ = torch.device("cuda:0")

    def padded(a):
        buf = torch.full((T + tail_rows, F), fill, dtype=torch.bfloat16, device=dev_)
        buf[:T] = t_act(a.reshape(T, F), w.dtype)
        return buf[:T].view(T, w.heads, w.d)

    q, k, v = padded(w.q), padded(w.k), padded(w.v)
    out = hs.attn_fwd(t_i32(w.offsets), T, t_i64(w.ts), q, k, v, t_f32(w.rab_p), t_f32(w.rab_t), w.n_max)
    torch.cuda.synchronize()
    return out


def test_fwd_causality_and_neighbours_bitwise():
    w = small(17, [260, 190, 70])
    base, _, _ = run_fwd(w)
    # perturb token j* of sequence 0 (and its time): earlier rows unchanged
    j = 150
    w2 = small(17, [260, 190, 70])
    w2.q[j] += 1.0
    w2.k[j] -= 2.0
    w2.v[j] *= 3.0
    w2.ts[j:260] += 1000
    pert, _, _ = run_fwd(w2)
    assert torch.equal(pert[:j], base[:j])
    assert not torch.equal(pert[j:260], base[j:260])
    # NaN in the other sequences' Q, K, V and in the rows past the last
    # token: sequence 1 unchanged bit for bit (a masked read of a NaN would
    # give 0 * NaN = NaN, so any such read shows)
    w3 = small(17, [260, 190, 70])
    for a in (w3.q, w3.k, w3.v):
        a[:260] = np.nan
        a[450:] = np.nan
    g3 = run_fwd_padded(w3)
    assert torch.equal(g3[260:450], base[260:450])
    assert not torch.isnan(g3[260:450].float()).any()
    # the first and last sequences alone, with NaN rows past T
    w4 = small(17, [260, 190, 70])
    for a in (w4.q, w4.k, w4.v):
        a[260:] = np.nan
    g4 = run_fwd_padded(w4)
    assert torch.equal(g4[:260], base[:260])


def test_fwd_deterministic():
    w = small(18, [500, 129])
    a, _, _ = run_fwd(w)
    b, _, _ = run_fwd(w)
    assert torch.equal(a, b)


def test_fwd_fp32_tiny_layer_attention():
    """fp32 path (d = 32, H = 2) on the tiny layer's shapes, tolerance 1e-4."""
    L = np.array([17, 64, 33, 5])
    w = synth.attention_workload("f32", 0, L, heads=2, d=32, n_max=64, dtype="f32", epilogue=True, act_std=1.0)
    out, _, _ = run_fwd(w, epilogue=False)
    ref, _ = ref_fwd(w, epilogue=False)
    assert rel_err(host(out), ref) <= F32_TOL
    out, _, _ = run_fwd(w, epilogue=True)
    ref, _ = ref_fwd(w, epilogue=True)
    assert rel_err(host(out), ref) <= F32_TOL


def test_fwd_full_size_1k_every_row():
    """B=32, lengths U{64..1024}, N_max=1024, H=4, d=128, no epilogue: the
    full launch, every element against the oracle."""
    w = synth.attn_fwd_1k()
    out, osv, _ = run_fwd(w, o_save=True)
    ref, _ = ref_fwd(w)
    err = rel_err(host(out), ref)
    err32 = rel_err(host(osv), ref)
    print("1k rel err bf16 out", err, "bound", bf16_bound(ref), "fp32 O", err32)
    assert err32 <= BF16_TOL
    assert err <= bf16_bound(ref)


@pytest.mark.timeout(900)
def test_fwd_full_size_8k_epilogue_every_row():
    """B=8, SL(1.6) lengths at N_max=8192, H=4, d=128 with LayerNorm(AV)*U:
    the full launch, every element of G and of the fp32 O against the
    oracle (about 180 GFLOP of fp64 on the host)."""
    w = synth.attn_8k(with_grad=False)
    out, osv, lst = run_fwd(w, o_save=True, stats=True)
    G, O = ref_fwd(w)
    e1 = rel_err(host(out), G)
    e2 = rel_err(host(osv), O)
    _, st = oracle.ln_gate(O, w.u, w.ln_eps)
    e3 = rel_err(host(lst)[:, 1], st[:, 1])
    print("8k rel err G", e1, "bound", bf16_bound(G), "O", e2, "rstd", e3)
    assert e2 <= BF16_TOL
    assert e1 <= bf16_bound(G)
    assert e3 <= BF16_TOL


def test_fwd_8k_deterministic():
    """The full 8k launch twice (split items, the gate): bit-identical."""
    w = synth.attn_8k(with_grad=False)
    a, oa, _ = run_fwd(w, o_save=True)
    b, ob, _ = run_fwd(w, o_save=True)
    assert torch.equal(a, b) and torch.equal(oa, ob)
