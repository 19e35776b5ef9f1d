"""Pins of the CPU oracle to things other than itself (no GPU).

Each test ties one part of the oracle to the pages' definitions (paper review
"Actions Speak Louder than Words", section 3, Eq. 1-3, M-FALCON) through
brute force, a closed form, an invariant, finite differences or a library
routine.  tests/test_oracle_mutants.py checks that plausible mistakes planted
in the oracle source make at least one of these fail.
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle
import synth
from brute import bucket_bitlen, dense_attn, dense_layer, dense_ln_gate


def silu(x):
    return x * expit(x)


def rand_case(rng, B=None, Lmax=40, H=None, d=None, n_max=None, monotone_ts=False, sparse_len=False):
    B = B or int(rng.integers(1, 6))
    H = H or int(rng.integers(1, 4))
    d = d or int(rng.choice([1, 2, 8, 32]))
    lengths = rng.integers(0 if sparse_len else 1, Lmax + 1, size=B)
    off = synth.offsets_of(lengths)
    T = int(off[-1])
    N = n_max or int(max(1, lengths.max()) + rng.integers(0, 8))
    if monotone_ts:
        ts = synth.timestamps(rng, lengths)
    else:
        ts = rng.integers(-10 ** 6, 10 ** 6, size=T).astype(np.int64) + synth.EPOCH
    q = rng.standard_normal((T, H, d))
    k = rng.standard_normal((T, H, d))
    v = rng.standard_normal((T, H, d))
    rab_p = rng.standard_normal((H, 2 * N + 1))
    rab_t = rng.standard_normal((H, 128))
    return dict(off=off, ts=ts, q=q, k=k, v=v, rab_p=rab_p, rab_t=rab_t, N=N, H=H, d=d, lengths=lengths)


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("seed", range(40))
def test_fwd_matches_dense_bruteforce(seed):
    rng = np.random.default_rng(1000 + seed)
    c = rand_case(rng, sparse_len=(seed % 5 == 0), monotone_ts=(seed % 2 == 0))
    got = oracle.attn_fwd(c["off"], c["ts"], c["q"], c["k"], c["v"], c["rab_p"], c["rab_t"], c["N"])
    ref = dense_attn(c["off"], c["ts"], c["q"], c["k"], c["v"], c["rab_p"], c["rab_t"], c["N"])
    scale = max(1e-300, np.abs(ref).max())
    assert np.abs(got - ref).max() <= 1e-12 * scale


def test_fwd_tiny_layer_workload_matches_dense():
    w = synth.tiny_layer_f32()
    lay = w.layers[0]
    got = oracle.layer_fwd(w.offsets, w.ts, w.x, lay, w.heads, w.d, w.n_max)
    ref, _, _ = dense_layer(w.offsets, w.ts, w.x, lay, w.heads, w.d, w.n_max)
    assert np.abs((got - w.x) - (ref - w.x)).max() <= 1e-12 * np.abs(ref - w.x).max()


@pytest.mark.parametrize("phi1", [0, 1])
def test_layer_matches_dense_strong_branch(phi1):
    """Strong-branch weights (std 1/sqrt(fan_in)) so Y - X is not swamped by
    the residual, and V scaled so the LayerNorm is not eps-dominated."""
    rng = np.random.default_rng(7 + phi1)
    H, d, D, N = 2, 8, 24, 16
    lengths = np.array([5, 16, 1, 9])
    off = synth.offsets_of(lengths)
    ts = synth.timestamps(rng, lengths)
    lay = synth.Layer(w1=rng.standard_normal((4 * H * d, D)) / math.sqrt(D), b1=rng.standard_normal(4 * H * d) * .1,
                      w2=rng.standard_normal((D, H * d)) / math.sqrt(H * d), b2=rng.standard_normal(D) * .1,
                      rab_p=rng.standard_normal((H, 2 * N + 1)), rab_t=rng.standard_normal((H, 128)))
    x = rng.standard_normal((int(off[-1]), D))
    got = oracle.layer_fwd(off, ts, x, lay, H, d, N, phi1=phi1)
    ref, _, _ = dense_layer(off, ts, x, lay, H, d, N, phi1=phi1)
    assert np.abs(got - ref).max() <= 1e-11 * np.abs(ref - x).max()


def test_layer_is_affine_in_w2_and_b2():
    """Two linear layers per block (review §5, encoder efficiency): Y - X
    depends on (W2, b2) only through G W2^T + b2, so it is linear in (W2, b2)."""
    rng = np.random.default_rng(3)
    H, d, D, N = 2, 4, 8, 8
    lengths = np.array([6, 3])
    off = synth.offsets_of(lengths)
    ts = synth.timestamps(rng, lengths)
    base = dict(w1=rng.standard_normal((4 * H * d, D)), b1=np.zeros(4 * H * d), rab_p=rng.standard_normal((H, 2 * N + 1)),
                rab_t=rng.standard_normal((H, 128)))
    x = rng.standard_normal((9, D))
    w2a, w2b = rng.standard_normal((D, H * d)), rng.standard_normal((D, H * d))
    b2a, b2b = rng.standard_normal(D), rng.standard_normal(D)
    ya = oracle.layer_fwd(off, ts, x, synth.Layer(w2=w2a, b2=b2a, **base), H, d, N) - x
    yb = oracle.layer_fwd(off, ts, x, synth.Layer(w2=w2b, b2=b2b, **base), H, d, N) - x
    yab = oracle.layer_fwd(off, ts, x, synth.Layer(w2=2 * w2a - w2b, b2=2 * b2a - b2b, **base), H, d, N) - x
    assert np.allclose(yab, 2 * ya - yb, rtol=1e-10, atol=1e-10)


# ---------------------------------------------------------------- closed forms

def test_closed_form_prefix_sum():
    """Q = 0, no time term, rab_p = c everywhere: s_ij = c, so
    O_i = SiLU(c)/N * sum_{j<=i} v_j -- a prefix sum."""
    rng = np.random.default_rng(5)
    H, d, N = 2, 3, 32
    lengths = np.array([7, 1, 20])
    off = synth.offsets_of(lengths)
    T = int(off[-1])
    c = 0.75
    q = np.zeros((T, H, d))
    k = rng.standard_normal((T, H, d))
    v = rng.standard_normal((T, H, d))
    rab_p = np.full((H, 2 * N + 1), c)
    got = oracle.attn_fwd(off, None, q, k, v, rab_p, None, N)
    sc = c / (1 + math.exp(-c)) / N
    for b in range(3):
        o, e = off[b], off[b + 1]
        ref = np.cumsum(v[o:e], axis=0).reshape(e - o, H * d) * sc
        assert np.allclose(got[o:e], ref, rtol=1e-13, atol=1e-15)


def test_closed_form_single_token():
    """L = 1: O_0 = SiLU(q.k + rab_p[N] + rab_t[0]) v / N."""
    rng = np.random.default_rng(6)
    H, d, N = 3, 5, 4
    off = np.array([0, 1])
    q, k, v = (rng.standard_normal((1, H, d)) for _ in range(3))
    rab_p = rng.standard_normal((H, 2 * N + 1))
    rab_t = rng.standard_normal((H, 128))
    got = oracle.attn_fwd(off, np.array([synth.EPOCH]), q, k, v, rab_p, rab_t, N)
    for h in range(H):
        s = float(q[0, h] @ k[0, h]) + rab_p[h, N] + rab_t[h, 0]
        assert np.allclose(got[0, h * d:(h + 1) * d], silu(s) * v[0, h] / N, rtol=1e-14, atol=0)


def test_zero_query_zero_tables_give_zero():
    """SiLU(0) = 0: with Q = 0 and zero tables every output is exactly 0."""
    rng = np.random.default_rng(8)
    c = rand_case(rng)
    z = np.zeros_like(c["rab_p"]), np.zeros_like(c["rab_t"])
    got = oracle.attn_fwd(c["off"], c["ts"], np.zeros_like(c["q"]), c["k"], c["v"], z[0], z[1], c["N"])
    assert np.all(got == 0.0)


def test_linear_in_v():
    rng = np.random.default_rng(9)
    c = rand_case(rng)
    v2 = rng.standard_normal(c["v"].shape)
    f = lambda v: oracle.attn_fwd(c["off"], c["ts"], c["q"], c["k"], v, c["rab_p"], c["rab_t"], c["N"])
    assert np.allclose(f(2.0 * c["v"] - 3.0 * v2), 2.0 * f(c["v"]) - 3.0 * f(v2), rtol=1e-11, atol=1e-12)


def test_bias_readout_closed_form():
    """Q = K = 0 and V = identity read every bias entry out:
    O_i[j] = SiLU(rab_p[j - i] + rab_t[bucket(t_i - t_j)]) / N for j <= i.
    With rab_p[j - i] = 1e-3 (j - i) + 0.05 h, rab_t[b] = 0.1 b - 0.02 h and
    t_j = 2^j - 1, the bucket floor(log2(t_i - t_j + 1)) is 0 on the diagonal,
    i for j = 0 and i - 1 for 0 < j < i."""
    L, H, N = 40, 2, 48
    off = np.array([0, L])
    ts = np.array([(1 << j) - 1 for j in range(L)], np.int64)
    q = np.zeros((L, H, 1))
    k = np.zeros((L, H, 1))
    v = np.tile(np.eye(L)[:, None, :], (1, H, 1))
    rel = np.arange(2 * N + 1) - N
    rab_p = np.stack([1e-3 * rel + 0.05 * h for h in range(H)])
    rab_t = np.stack([0.1 * np.arange(128) - 0.02 * h for h in range(H)])
    got = oracle.attn_fwd(off, ts, q, k, v, rab_p, rab_t, N)
    for i in range(L):
        for h in range(H):
            for j in range(L):
                if j > i:
                    ref = 0.0
                else:
                    bk = 0 if j == i else (i if j == 0 else i - 1)
                    s = 1e-3 * (j - i) + 0.05 * h + 0.1 * bk - 0.02 * h
                    ref = silu(s) / N
                assert abs(got[i, h * L + j] - ref) <= 1e-15, (i, h, j)


def test_time_bucket_exhaustive_and_powers():
    for dt in list(range(0, 70000)) + [-x for x in range(1, 5000)]:
        assert oracle.time_bucket(dt) == bucket_bitlen(dt), dt
    for e in range(1, 63):
        for dt in ((1 << e) - 2, (1 << e) - 1, 1 << e):
            for sgn in (1, -1):
                assert oracle.time_bucket(sgn * dt) == bucket_bitlen(dt), (e, dt)


def test_position_clip_beyond_n_max():
    """A sequence longer than N_max exercises clip(j - i, -N, N): against
    brute force (which clips with numpy)."""
    rng = np.random.default_rng(11)
    c = rand_case(rng, B=2, Lmax=30, H=2, d=4, n_max=6)
    got = oracle.attn_fwd(c["off"], c["ts"], c["q"], c["k"], c["v"], c["rab_p"], c["rab_t"], 6)
    ref = dense_attn(c["off"], c["ts"], c["q"], c["k"], c["v"], c["rab_p"], c["rab_t"], 6)
    assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max()


def test_row_subset_equals_full():
    rng = np.random.default_rng(12)
    c = rand_case(rng, B=4, Lmax=30)
    full = oracle.attn_fwd(c["off"], c["ts"], c["q"], c["k"], c["v"], c["rab_p"], c["rab_t"], c["N"])
    rows = rng.choice(int(c["off"][-1]), size=min(10, int(c["off"][-1])), replace=False)
    sub = oracle.attn_fwd(c["off"], c["ts"], c["q"], c["k"], c["v"], c["rab_p"], c["rab_t"], c["N"], rows=rows)
    assert np.array_equal(sub, full[rows])


# ---------------------------------------------------------------- invariants

def test_causality_bitwise():
    """Changing token j* (its q, k, v and time) leaves every earlier output of
    its sequence bit-identical."""
    rng = np.random.default_rng(13)
    c = rand_case(rng, B=3, Lmax=30, monotone_ts=True)
    base = oracle.attn_fwd(c["off"], c["ts"], c["q"], c["k"], c["v"], c["rab_p"], c["rab_t"], c["N"])
    b = int(np.argmax(c["lengths"]))
    o, e = int(c["off"][b]), int(c["off"][b + 1])
    jstar = o + (e - o) // 2
    q, k, v, ts = c["q"].copy(), c["k"].copy(), c["v"].copy(), c["ts"].copy()
    q[jstar] += 5.0
    k[jstar] -= 3.0
    v[jstar] *= -7.0
    ts[jstar] += 12345
    pert = oracle.attn_fwd(c["off"], ts, q, k, v, c["rab_p"], c["rab_t"], c["N"])
    assert np.array_equal(pert[o:jstar], base[o:jstar])
    assert not np.array_equal(pert[jstar:e], base[jstar:e])


def test_neighbour_and_batch_invariance():
    """Sequence b's output does not depend on other sequences (garbage there),
    equals its own B = 1 run, and permuting sequences permutes outputs."""
    rng = np.random.default_rng(14)
    c = rand_case(rng, B=4, Lmax=25, monotone_ts=True)
    off = c["off"]
    base = oracle.attn_fwd(off, c["ts"], c["q"], c["k"], c["v"], c["rab_p"], c["rab_t"], c["N"])
    for b in range(4):
        o, e = int(off[b]), int(off[b + 1])
        q, k, v = c["q"].copy(), c["k"].copy(), c["v"].copy()
        mask = np.ones(len(q), bool)
        mask[o:e] = False
        q[mask], k[mask], v[mask] = 1e30, -1e30, 1e30
        g = oracle.attn_fwd(off, c["ts"], q, k, v, c["rab_p"], c["rab_t"], c["N"])
        assert np.array_equal(g[o:e], base[o:e])
        single = oracle.attn_fwd(np.array([0, e - o]), c["ts"][o:e], c["q"][o:e], c["k"][o:e], c["v"][o:e],
                                 c["rab_p"], c["rab_t"], c["N"])
        assert np.array_equal(single, base[o:e])
    perm = [2, 0, 3, 1]
    idx = np.concatenate([np.arange(off[b], off[b + 1]) for b in perm])
    poff = synth.offsets_of(c["lengths"][perm])
    p = oracle.attn_fwd(poff, c["ts"][idx], c["q"][idx], c["k"][idx], c["v"][idx], c["rab_p"], c["rab_t"], c["N"])
    assert np.array_equal(p, base[idx])


# ---------------------------------------------------------------- epilogue

def test_ln_gate_against_library_and_moments():
    rng = np.random.default_rng(15)
    T, F, eps = 37, 64, 1e-5
    O = rng.standard_normal((T, F)) * rng.uniform(1e-4, 3, size=(T, 1)) + rng.standard_normal((T, 1))
    U = rng.standard_normal((T, F))
    G, st = oracle.ln_gate(O, U, eps)
    assert np.allclose(G, dense_ln_gate(O, U, eps), rtol=1e-12, atol=1e-12)
    xh, _ = oracle.ln_gate(O, np.ones_like(O), eps)
    var = O.var(axis=1)
    assert np.allclose(xh.mean(axis=1), 0, atol=1e-12)
    assert np.allclose((xh ** 2).mean(axis=1), var / (var + eps), rtol=1e-12)
    assert np.allclose(st[:, 0], O.mean(axis=1), rtol=1e-13, atol=1e-13)
    assert np.allclose(st[:, 1], 1 / np.sqrt(var + eps), rtol=1e-12)


# ---------------------------------------------------------------- backward

def _loss(c, U, dG, q, k, v, u, rp, rt, eps):
    O = oracle.attn_fwd(c["off"], c["ts"], q, k, v, rp, rt, c["N"])
    if U is None:
        return float((O * dG).sum())
    G, _ = oracle.ln_gate(O, u, eps)
    return float((G * dG).sum())


@pytest.mark.parametrize("with_u", [True, False])
def test_bwd_finite_differences(with_u):
    """Central differences of the fp64 forward (step 1e-6) against every
    analytic gradient: dq, dk, dv, du, drab_p, drab_t."""
    rng = np.random.default_rng(16 + with_u)
    H, d, N = 2, 3, 8
    lengths = np.array([5, 3])
    off = synth.offsets_of(lengths)
    T = 8
    ts = synth.timestamps(rng, lengths)
    c = dict(off=off, ts=ts, N=N)
    q, k = rng.standard_normal((T, H, d)), rng.standard_normal((T, H, d))
    v = rng.standard_normal((T, H, d)) * 8.0
    u = rng.standard_normal((T, H * d)) if with_u else None
    rp, rt = rng.standard_normal((H, 2 * N + 1)), rng.standard_normal((H, 128)) * 0.5
    dG = rng.standard_normal((T, H * d))
    eps = 1e-3
    g = oracle.attn_bwd(off, ts, q, k, v, rp, rt, N, u, eps, dG)
    args = dict(q=q, k=k, v=v, u=u, rp=rp, rt=rt)
    names = dict(q="dq", k="dk", v="dv", u="du", rp="drab_p", rt="drab_t")
    h = 1e-6
    for name, grad_name in names.items():
        if args[name] is None:
            continue
        base = args[name]
        num = np.zeros_like(base)
        it = np.nditer(base, flags=["multi_index"])
        for _ in it:
            ix = it.multi_index
            a2 = dict(args)
            p, m = base.copy(), base.copy()
            p[ix] += h
            m[ix] -= h
            a2[name] = p
            fp = _loss(c, u, dG, a2["q"], a2["k"], a2["v"], a2["u"], a2["rp"], a2["rt"], eps)
            a2[name] = m
            fm = _loss(c, u, dG, a2["q"], a2["k"], a2["v"], a2["u"], a2["rp"], a2["rt"], eps)
            num[ix] = (fp - fm) / (2 * h)
        ana = g[grad_name]
        err = np.abs(num - ana).max() / max(1e-12, np.abs(ana).max())
        assert err < 1e-6, (name, err)


@pytest.mark.parametrize("with_u", [True, False])
def test_bwd_dq_rows_equal_full_backward(with_u):
    rng = np.random.default_rng(22)
    c = rand_case(rng, B=3, Lmax=20, H=2, d=4, monotone_ts=True)
    T = int(c["off"][-1])
    U = rng.standard_normal((T, c["H"] * c["d"])) if with_u else None
    dG = rng.standard_normal((T, c["H"] * c["d"]))
    g = oracle.attn_bwd(c["off"], c["ts"], c["q"], c["k"], c["v"], c["rab_p"], c["rab_t"], c["N"], U, 1e-5, dG)
    rows = rng.choice(T, size=min(7, T), replace=False)
    sub = oracle.attn_bwd_dq_rows(c["off"], c["ts"], c["q"], c["k"], c["v"], c["rab_p"], c["rab_t"], c["N"], U, 1e-5,
                                  dG, rows)
    assert np.allclose(sub, g["dq"][rows], rtol=1e-12, atol=1e-12)


def test_bwd_identities():
    """Every ds_ij lands once in each table: sum(drab_p[h]) = sum(drab_t[h]);
    and sum_i dq_i . q_i = sum_j dk_j . k_j per head (both = sum ds_ij q_i.k_j)."""
    rng = np.random.default_rng(18)
    c = rand_case(rng, B=3, Lmax=20, H=2, d=4, monotone_ts=True)
    U = rng.standard_normal((int(c["off"][-1]), c["H"] * c["d"]))
    dG = rng.standard_normal(U.shape)
    g = oracle.attn_bwd(c["off"], c["ts"], c["q"], c["k"], c["v"], c["rab_p"], c["rab_t"], c["N"], U, 1e-5, dG)
    for h in range(c["H"]):
        a, b = g["drab_p"][h].sum(), g["drab_t"][h].sum()
        assert abs(a - b) <= 1e-10 * max(1.0, abs(a))
        x = (g["dq"][:, h] * c["q"][:, h]).sum()
        y = (g["dk"][:, h] * c["k"][:, h]).sum()
        assert abs(x - y) <= 1e-10 * max(1.0, abs(x))


def _layer_case(rng, phi1):
    H, d, D, N = 2, 3, 5, 6
    lengths = np.array([4, 3])
    off = synth.offsets_of(lengths)
    ts = synth.timestamps(rng, lengths)
    lay = dict(w1=rng.standard_normal((4 * H * d, D)), b1=rng.standard_normal(4 * H * d) * .5,
               w2=rng.standard_normal((D, H * d)), b2=rng.standard_normal(D),
               rab_p=rng.standard_normal((H, 2 * N + 1)), rab_t=rng.standard_normal((H, 128)) * .5)
    x = rng.standard_normal((int(off[-1]), D))
    dy = rng.standard_normal(x.shape)
    return H, d, D, N, off, ts, lay, x, dy


@pytest.mark.parametrize("phi1", [0, 1])
def test_layer_bwd_finite_differences(phi1):
    """Central differences of the fp64 layer forward (step 1e-6) of the loss
    sum(dY * Y) against every analytic gradient of the layer backward: dx,
    dw1, db1, dw2, db2, drab_p, drab_t."""
    rng = np.random.default_rng(40 + phi1)
    H, d, D, N, off, ts, lay, x, dy = _layer_case(rng, phi1)
    eps = 1e-3
    g = oracle.layer_bwd(off, ts, x, synth.Layer(**lay), dy, H, d, N, phi1=phi1, eps=eps)

    def loss(xx, params):
        return float((oracle.layer_fwd(off, ts, xx, synth.Layer(**params), H, d, N, phi1=phi1, eps=eps) * dy).sum())

    h = 1e-6
    grads = dict(x="dx", w1="dw1", b1="db1", w2="dw2", b2="db2", rab_p="drab_p", rab_t="drab_t")
    for name, gname in grads.items():
        base = x if name == "x" else lay[name]
        num = np.zeros_like(base)
        it = np.nditer(base, flags=["multi_index"])
        for _ in it:
            ix = it.multi_index
            vals = []
            for sgn in (1, -1):
                pert = base.copy()
                pert[ix] += sgn * h
                if name == "x":
                    vals.append(loss(pert, lay))
                else:
                    vals.append(loss(x, dict(lay, **{name: pert})))
            num[ix] = (vals[0] - vals[1]) / (2 * h)
        ana = g[gname]
        err = np.abs(num - ana).max() / max(1e-12, np.abs(ana).max())
        assert err < 1e-6, (name, err)


def test_layer_bwd_residual_and_bias_identities():
    """With W2 = 0 the layer is Y = X + b2: dX = dY exactly, every other
    weight gradient but dW2 and db2 vanishes, db2 = column sums of dY.  And
    db1 is dW1 of a constant-one input column: appending a unit column to X
    (a zero column to W1, a zero row to W2, a zero entry to b2 and dY) makes
    that column of dW1 equal db1."""
    rng = np.random.default_rng(44)
    H, d, D, N, off, ts, lay, x, dy = _layer_case(rng, 0)
    g = oracle.layer_bwd(off, ts, x, synth.Layer(**dict(lay, w2=np.zeros_like(lay["w2"]))), dy, H, d, N)
    assert np.array_equal(g["dx"], dy)
    assert not g["dw1"].any() and not g["db1"].any() and not g["drab_p"].any() and not g["drab_t"].any()
    assert np.allclose(g["db2"], dy.sum(axis=0), rtol=1e-13, atol=1e-13)
    x1 = np.concatenate([x, np.ones((x.shape[0], 1))], axis=1)
    w1 = np.concatenate([lay["w1"], np.zeros((lay["w1"].shape[0], 1))], axis=1)
    lay2 = dict(lay, w1=w1, w2=np.concatenate([lay["w2"], np.zeros((1, H * d))], axis=0), b2=np.append(lay["b2"], 0.))
    dy1 = np.concatenate([dy, np.zeros((x.shape[0], 1))], axis=1)
    g2 = oracle.layer_bwd(off, ts, x1, synth.Layer(**lay2), dy1, H, d, N)
    assert np.allclose(g2["dw1"][:, D], g2["db1"], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- M-FALCON

def test_mfalcon_equals_last_row_of_full_forward():
    """A candidate scored against the cache equals the last row of the full
    causal layer stack run on [history; candidate] -- the cache only removes
    recomputation (review §3, M-FALCON)."""
    rng = np.random.default_rng(19)
    H, d, D, N, L = 2, 4, 12, 16, 2
    hist = np.array([5, 7, 0])
    hoff = synth.offsets_of(hist)
    hts = synth.timestamps(rng, hist)
    layers = [synth.Layer(w1=rng.standard_normal((4 * H * d, D)) / math.sqrt(D), b1=rng.standard_normal(4 * H * d) * .1,
                          w2=rng.standard_normal((D, H * d)) / math.sqrt(H * d), b2=rng.standard_normal(D) * .1,
                          rab_p=rng.standard_normal((H, 2 * N + 1)), rab_t=rng.standard_normal((H, 128)))
              for _ in range(L)]
    xh = rng.standard_normal((int(hoff[-1]), D))
    ncand = np.array([3, 2, 2])
    coff = synth.offsets_of(ncand)
    cts = np.array([hts[hoff[1] - 1] + 17, hts[hoff[2] - 1] + 1, synth.EPOCH + 5], np.int64)
    xc = rng.standard_normal((int(coff[-1]), D))
    kv = oracle.history_cache(hoff, hts, xh, layers, H, d, N)
    y = oracle.mfalcon(hoff, hts, coff, cts, layers, kv, xc, H, d, N)
    for u in range(3):
        for c in range(coff[u], coff[u + 1]):
            seq_x = np.concatenate([xh[hoff[u]:hoff[u + 1]], xc[c:c + 1]])
            seq_t = np.concatenate([hts[hoff[u]:hoff[u + 1]], cts[u:u + 1]])
            h = seq_x
            for lay in layers:
                h = oracle.layer_fwd(np.array([0, len(seq_x)]), seq_t, h, lay, H, d, N)
            assert np.allclose(y[c], h[-1], rtol=1e-12, atol=1e-12), (u, c)


def test_layer_kv_equals_layer_forward_cache():
    """The cache-only layer (K, V of phi1(x W1^T + b1)) returns exactly the
    K and V the full layer forward keeps, for SiLU and ReLU."""
    rng = np.random.default_rng(23)
    H, d, D, N = 2, 4, 12, 16
    hist = np.array([5, 9])
    off = synth.offsets_of(hist)
    ts = synth.timestamps(rng, hist)
    lay = synth.Layer(w1=rng.standard_normal((4 * H * d, D)), b1=rng.standard_normal(4 * H * d),
                      w2=rng.standard_normal((D, H * d)), b2=rng.standard_normal(D),
                      rab_p=rng.standard_normal((H, 2 * N + 1)), rab_t=rng.standard_normal((H, 128)))
    x = rng.standard_normal((int(off[-1]), D))
    for phi1 in (0, 1):
        _, K, V = oracle.layer_fwd(off, ts, x, lay, H, d, N, phi1=phi1, return_kv=True)
        kv = oracle.layer_kv(x, lay, H, d, phi1=phi1)
        assert np.allclose(kv[0], K, rtol=1e-14, atol=1e-14) and np.allclose(kv[1], V, rtol=1e-14, atol=1e-14)


def test_layer_append_equals_full_forward():
    """Appending a_u new actions to a cached history gives exactly rows
    n_u.. of the layer run over the whole sequence [history; new] (the cache
    only removes recomputation), and the merged cache equals that run's K,
    V.  Users with no history, no new actions, one new action and several."""
    rng = np.random.default_rng(24)
    H, d, D, N = 2, 4, 12, 16
    hist = np.array([5, 0, 9, 4, 7])
    add = np.array([3, 4, 1, 0, 6])
    hoff, aoff = synth.offsets_of(hist), synth.offsets_of(add)
    lay = synth.Layer(w1=rng.standard_normal((4 * H * d, D)) / math.sqrt(D), b1=rng.standard_normal(4 * H * d) * .1,
                      w2=rng.standard_normal((D, H * d)) / math.sqrt(H * d), b2=rng.standard_normal(D) * .1,
                      rab_p=rng.standard_normal((H, 2 * N + 1)), rab_t=rng.standard_normal((H, 128)))
    full_len = hist + add
    ts_full = synth.timestamps(rng, full_len)
    x_full = rng.standard_normal((int(full_len.sum()), D))
    foff = synth.offsets_of(full_len)
    hrows = np.concatenate([np.arange(foff[u], foff[u] + hist[u]) for u in range(len(hist))])
    arows = np.concatenate([np.arange(foff[u] + hist[u], foff[u + 1]) for u in range(len(hist))])
    _, Kh, Vh = oracle.layer_fwd(hoff, ts_full[hrows], x_full[hrows], lay, H, d, N, return_kv=True)
    y_new, kv_out = oracle.layer_append(hoff, ts_full[hrows], aoff, ts_full[arows], lay, np.stack([Kh, Vh]),
                                        x_full[arows], H, d, N)
    y_full, Kf, Vf = oracle.layer_fwd(foff, ts_full, x_full, lay, H, d, N, return_kv=True)
    assert np.allclose(y_new, y_full[arows], rtol=1e-12, atol=1e-12)
    assert np.allclose(kv_out[0], Kf, rtol=1e-12, atol=1e-12) and np.allclose(kv_out[1], Vf, rtol=1e-12, atol=1e-12)


def test_mfalcon_candidates_independent():
    """A candidate's score does not depend on the other candidates."""
    rng = np.random.default_rng(20)
    H, d, D, N = 2, 4, 8, 8
    hist = np.array([6])
    hoff = synth.offsets_of(hist)
    hts = synth.timestamps(rng, hist)
    layers = [synth.Layer(w1=rng.standard_normal((4 * H * d, D)) * .3, b1=np.zeros(4 * H * d),
                          w2=rng.standard_normal((D, H * d)) * .3, b2=np.zeros(D),
                          rab_p=rng.standard_normal((H, 2 * N + 1)), rab_t=rng.standard_normal((H, 128)))]
    kv = oracle.history_cache(hoff, hts, rng.standard_normal((6, D)), layers, H, d, N)
    xc = rng.standard_normal((4, D))
    cts = np.array([hts[-1] + 3])
    y = oracle.mfalcon(hoff, hts, np.array([0, 4]), cts, layers, kv, xc, H, d, N)
    xc2 = xc.copy()
    xc2[1:] = rng.standard_normal((3, D)) * 10
    y2 = oracle.mfalcon(hoff, hts, np.array([0, 4]), cts, layers, kv, xc2, H, d, N)
    assert np.array_equal(y[0], y2[0])


# ---------------------------------------------------------------- inputs

def test_stochastic_length_mean():
    """E[min(n, ceil(n u^(1/a)))] = n a/(a+1) + (about 1/2 from the ceiling)."""
    rng = np.random.default_rng(21)
    L = synth.stochastic_lengths(rng, 200000, 4096, 1.6)
    assert abs(L.mean() - (4096 * 1.6 / 2.6 + 0.5)) < 6.0
    assert L.min() >= 1 and L.max() <= 4096


def test_inputs_deterministic():
    a, b = synth.attn_fwd_1k(), synth.attn_fwd_1k()
    assert np.array_equal(a.q, b.q) and np.array_equal(a.ts, b.ts) and np.array_equal(a.rab_p, b.rab_p)
    w = synth.tiny_layer_f32()
    assert list(w.lengths) == [17, 64, 33, 5] and w.total == 119


# ---------------------------------------------------------------- softmax comparator

def test_softmax_comparator_against_library_softmax():
    """The comparator equals a dense formulation built from scipy's softmax
    with an explicit causal mask, on random tiny ragged batches."""
    from scipy.special import softmax
    rng = np.random.default_rng(30)
    for trial in range(10):
        L = rng.integers(0, 9, size=rng.integers(1, 4))
        H, d = int(rng.integers(1, 3)), int(rng.choice([1, 4, 8]))
        off = synth.offsets_of(L)
        T = int(off[-1])
        q, k, v = (rng.standard_normal((T, H, d)) for _ in range(3))
        got, lse = oracle.softmax_attn_fwd(off, q, k, v, want_lse=True)
        for b in range(len(L)):
            o, n = int(off[b]), int(L[b])
            for h in range(H):
                S = q[o:o + n, h] @ k[o:o + n, h].T / math.sqrt(d)
                S = np.where(np.tril(np.ones((n, n), bool)), S, -np.inf)
                P = softmax(S, axis=1) if n else S
                ref = P @ v[o:o + n, h] if n else np.zeros((0, d))
                assert np.allclose(got[o:o + n, h * d:(h + 1) * d], ref, rtol=1e-12, atol=1e-12)
                if n:
                    m = S.max(axis=1)
                    assert np.allclose(lse[o:o + n, h], m + np.log(np.exp(S - m[:, None]).sum(axis=1)), rtol=1e-12)


def test_softmax_comparator_closed_forms():
    """Q = 0: every key weighs the same, O_i is the mean of V_0..V_i (a
    prefix mean).  Adding one vector t to every key of a sequence shifts each
    row's scores by q_i.t and leaves O unchanged.  V = 1 gives O = 1."""
    rng = np.random.default_rng(31)
    L = np.array([7, 1, 12])
    off = synth.offsets_of(L)
    T, H, d = int(off[-1]), 2, 4
    q, k, v = (rng.standard_normal((T, H, d)) for _ in range(3))
    o0 = oracle.softmax_attn_fwd(off, np.zeros_like(q), k, v)
    for b in range(3):
        s, n = int(off[b]), int(L[b])
        pm = np.cumsum(v[s:s + n], axis=0) / np.arange(1, n + 1)[:, None, None]
        assert np.allclose(o0[s:s + n].reshape(n, H, d), pm, rtol=1e-12, atol=1e-12)
    base = oracle.softmax_attn_fwd(off, q, k, v)
    k2 = k.copy()
    for b in range(3):
        k2[off[b]:off[b + 1]] += rng.standard_normal((1, H, d)) * 3
    assert np.allclose(oracle.softmax_attn_fwd(off, q, k2, v), base, rtol=1e-10, atol=1e-10)
    assert np.allclose(oracle.softmax_attn_fwd(off, q, k, np.ones_like(v)), 1.0, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- Stochastic Length sampler

def test_sl_sample_selection_definition():
    """Against a sort-based statement of the same rule (numpy lexsort by key
    then position): the kept actions are the L with the smallest keys, in
    input order, with L = max(1, min(n, ceil(n u^(1/alpha)))); duplicate
    keys (few distinct values) take the earlier positions first."""
    rng = np.random.default_rng(40)
    for trial in range(30):
        L = rng.integers(0, 40, size=rng.integers(1, 6))
        off = synth.offsets_of(L)
        keys = rng.integers(0, 6 if trial % 2 else 2 ** 32, size=int(off[-1]), dtype=np.uint64).astype(np.uint32)
        u = rng.random(len(L))
        alpha = float(rng.choice([1.2, 1.6, 2.0]))
        oo, idx = oracle.sl_sample(off, alpha, u, keys)
        want = []
        for b in range(len(L)):
            n = int(L[b])
            m = 0 if n == 0 else max(1, min(n, math.ceil(n * u[b] ** (1.0 / alpha))))
            kk = keys[off[b]:off[b + 1]]
            order = np.lexsort((np.arange(n), kk))[:m]
            want += sorted((off[b] + order).tolist())
            assert oo[b + 1] - oo[b] == m
        assert idx.tolist() == want


def test_sl_sample_law_and_uniformity():
    """u = 1 keeps everything and a tiny u keeps one action; over many draws
    the mean kept length is n alpha/(alpha+1) + ~1/2 (the law's closed form),
    and every position is kept with the same probability (uniform keys)."""
    n, alpha = 64, 1.6
    off = np.array([0, n], np.int32)
    keys = np.arange(n, dtype=np.uint32)
    oo, _ = oracle.sl_sample(off, alpha, [1.0], keys)
    assert oo[1] == n
    oo, _ = oracle.sl_sample(off, alpha, [1e-12], keys)
    assert oo[1] == 1
    rng = np.random.default_rng(41)
    trials = 4000
    B = trials
    offs = synth.offsets_of(np.full(B, n))
    oo, idx = oracle.sl_sample(offs, alpha, rng.random(B), rng.integers(0, 2 ** 32, size=B * n, dtype=np.uint64).astype(np.uint32))
    lens = np.diff(oo)
    assert abs(lens.mean() - (n * alpha / (alpha + 1) + 0.5)) < 1.0
    pos_counts = np.bincount(idx % n, minlength=n)
    expect = lens.sum() / n
    assert np.abs(pos_counts - expect).max() < 6 * np.sqrt(expect)
