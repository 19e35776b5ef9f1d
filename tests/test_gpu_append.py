"""GPU parity of hstu_layer_append (new actions appended to cached user
histories, one layer) through the C ABI against the fp64 oracle: the new
tokens' layer output and the merged K/V caches.  The oracle's append is
pinned to the full causal layer over [history; new] (test_oracle_pins)."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import BF16_TOL, bf16_bound, host, rel_err, round_bf16, t_act, t_f32, t_i32, t_i64

pytestmark = pytest.mark.gpu

hs = pytest.importorskip("hstu_sequential_transducer_amd")


def dev_layer(lay):
    return dict(w1=t_act(lay.w1, "bf16"), b1=t_f32(lay.b1), w2=t_act(lay.w2, "bf16"), b2=t_f32(lay.b2),
                rab_p=t_f32(lay.rab_p), rab_t=t_f32(lay.rab_t), phi1=0)


def strong(w, seed):
    rng = np.random.default_rng(seed)
    lay = w.layers[0]
    D, HD = w.d_model, w.heads * w.d
    lay.w1 = synth.round_bf16(rng.standard_normal(lay.w1.shape).astype(np.float32) / math.sqrt(D))
    lay.w2 = synth.round_bf16(rng.standard_normal(lay.w2.shape).astype(np.float32) / math.sqrt(HD))
    lay.rab_p = (rng.standard_normal(lay.rab_p.shape) * 0.5).astype(np.float32)
    lay.rab_t = (rng.standard_normal(lay.rab_t.shape) * 0.5).astype(np.float32)


def gpu_cache(w, lay, off, x, ts):
    """This layer's K, V of the history rows, built by hstu_layer_fwd."""
    T = int(off[-1])
    kc = torch.empty((T, w.heads * w.d), dtype=torch.bfloat16, device="cuda:0")
    vc = torch.empty_like(kc)
    if T:
        hs.layer_fwd(t_i32(off), T, t_i64(ts), t_act(x, "bf16"), lay, w.heads, w.d, w.n_max, k_cache=kc, v_cache=vc)
    return kc, vc


def gpu_append(w, lay, hoff, hts, kc, vc, aoff, ats, xn):
    y, ko, vo = hs.layer_append(t_i32(hoff), int(hoff[-1]), t_i64(hts), t_i32(aoff), int(aoff[-1]), t_i64(ats),
                                t_act(xn, "bf16"), lay, kc, vc, w.heads, w.d, w.n_max)
    torch.cuda.synchronize()
    return y, ko, vo


def branch_check(tag, y, ref, x):
    b = ref - x
    e = rel_err(y - x, b)
    bound = BF16_TOL + np.abs(round_bf16(ref) - ref).max() / np.sqrt(np.mean(b ** 2))
    e2 = rel_err(y, ref)
    print(tag, "y err", e2, "bound", bf16_bound(ref), "branch err", e, "bound", bound, flush=True)
    assert e2 <= bf16_bound(ref)
    assert e <= bound


@pytest.mark.parametrize("strong_w", [False, True])
def test_append_small_against_oracle(strong_w):
    """Six users: histories {100, 0, 300, 5, 129, 257}, new actions {3, 40,
    1, 0, 200, 130} (an empty history, an empty append, appends that cross
    query tiles), D=512, H=4, d=128, N_max=1024."""
    w = synth.append_workload("append-small", 91, [100, 0, 300, 5, 129, 257], [3, 40, 1, 0, 200, 130], n_max=1024)
    if strong_w:
        strong(w, 92)
    lay = w.layers[0]
    dl = dev_layer(lay)
    kc, vc = gpu_cache(w, dl, w.offsets, w.x, w.ts)
    y, ko, vo = gpu_append(w, dl, w.offsets, w.ts, kc, vc, w.add_offsets, w.add_ts, w.x_new)
    _, K, V = oracle.layer_fwd(w.offsets, w.ts, w.x, lay, w.heads, w.d, w.n_max, return_kv=True)
    ref, kv = oracle.layer_append(w.offsets, w.ts, w.add_offsets, w.add_ts, lay, np.stack([K, V]), w.x_new, w.heads,
                                  w.d, w.n_max)
    branch_check("append small strong=%s" % strong_w, host(y), ref, w.x_new)
    Tm = kv.shape[1]
    Kr, Vr = kv[0].reshape(Tm, -1), kv[1].reshape(Tm, -1)
    assert rel_err(host(ko), Kr) <= bf16_bound(Kr)
    assert rel_err(host(vo), Vr) <= bf16_bound(Vr)
    # the history rows of the merged caches are copies of the input caches
    for u in range(len(w.lengths)):
        h0, n = int(w.offsets[u]), int(w.lengths[u])
        m0 = h0 + int(w.add_offsets[u])
        assert torch.equal(ko[m0:m0 + n], kc[h0:h0 + n]) and torch.equal(vo[m0:m0 + n], vc[h0:h0 + n])


def test_append_twice_equals_oracle_stream():
    """Two appends in a row (the second reads the first's merged caches)
    match the oracle's two appends, which equal the full layer over
    [history; first; second]."""
    w = synth.append_workload("append-2", 93, [64, 500, 1], [10, 1, 130], n_max=1024)
    w2 = synth.append_workload("append-2b", 94, [74, 501, 131], [5, 77, 2], n_max=1024)
    lay = w.layers[0]
    dl = dev_layer(lay)
    kc, vc = gpu_cache(w, dl, w.offsets, w.x, w.ts)
    y1, ko, vo = gpu_append(w, dl, w.offsets, w.ts, kc, vc, w.add_offsets, w.add_ts, w.x_new)
    # the second append: its history is [history; first append], times as merged
    moff = w.offsets + w.add_offsets
    mts = np.concatenate([np.concatenate([w.ts[w.offsets[u]:w.offsets[u + 1]],
                                          w.add_ts[w.add_offsets[u]:w.add_offsets[u + 1]]]) for u in range(3)])
    ats2 = np.concatenate([mts[moff[u + 1] - 1] + 1 + np.arange(int(w2.add_offsets[u + 1] - w2.add_offsets[u])) * 37
                           for u in range(3)]).astype(np.int64)
    y2, ko2, vo2 = gpu_append(w, dl, moff, mts, ko, vo, w2.add_offsets, ats2, w2.x_new)
    _, K, V = oracle.layer_fwd(w.offsets, w.ts, w.x, lay, w.heads, w.d, w.n_max, return_kv=True)
    r1, kv1 = oracle.layer_append(w.offsets, w.ts, w.add_offsets, w.add_ts, lay, np.stack([K, V]), w.x_new, w.heads,
                                  w.d, w.n_max)
    r2, kv2 = oracle.layer_append(moff, mts, w2.add_offsets, ats2, lay, kv1, w2.x_new, w.heads, w.d, w.n_max)
    branch_check("append twice, first", host(y1), r1, w.x_new)
    branch_check("append twice, second", host(y2), r2, w2.x_new)
    Tm = kv2.shape[1]
    assert rel_err(host(ko2), kv2[0].reshape(Tm, -1)) <= bf16_bound(kv2[0])


def test_append_matches_full_forward_on_gpu():
    """On the GPU too, the appended rows agree with hstu_layer_fwd run on the
    whole sequences [history; new] (same kernels; the new rows' queries see
    the same key tiles in the same order)."""
    w = synth.append_workload("append-full", 95, [300, 129, 7], [40, 200, 1], n_max=512)
    lay = w.layers[0]
    dl = dev_layer(lay)
    kc, vc = gpu_cache(w, dl, w.offsets, w.x, w.ts)
    y, ko, vo = gpu_append(w, dl, w.offsets, w.ts, kc, vc, w.add_offsets, w.add_ts, w.x_new)
    U = len(w.lengths)
    full_len = w.lengths + np.diff(w.add_offsets)
    rows_h = [np.arange(w.offsets[u], w.offsets[u + 1]) for u in range(U)]
    rows_a = [np.arange(w.add_offsets[u], w.add_offsets[u + 1]) for u in range(U)]
    xf = np.concatenate([np.concatenate([w.x[rows_h[u]], w.x_new[rows_a[u]]]) for u in range(U)])
    tf = np.concatenate([np.concatenate([w.ts[rows_h[u]], w.add_ts[rows_a[u]]]) for u in range(U)])
    foff = synth.offsets_of(full_len)
    kf, vf = gpu_cache(w, dl, foff, xf, tf)
    yf = hs.layer_fwd(t_i32(foff), int(foff[-1]), t_i64(tf), t_act(xf, "bf16"), dl, w.heads, w.d, w.n_max)
    torch.cuda.synchronize()
    new_rows = np.concatenate([np.arange(foff[u] + w.lengths[u], foff[u + 1]) for u in range(U)])
    e = rel_err(host(y), host(yf)[new_rows])
    print("append vs full forward on the GPU: y", e, flush=True)
    assert e <= 1e-2
    assert rel_err(host(ko), host(kf)) <= 1e-2 and rel_err(host(vo), host(vf)) <= 1e-2


@pytest.mark.timeout(600)
def test_append_64_users_sl_histories():
    """64 users with Stochastic-Length histories (n = 4096, alpha 1.6) and 16
    new actions each, N_max = 4096: the full launch; the oracle checks 12
    users (every fifth by history length, from the shortest to the
    longest), whose caches it builds itself."""
    m = synth.mfalcon_64users()
    adds = np.full(64, 16)
    w = synth.append_workload("append-64", 96, m.lengths, adds, n_max=4096)
    lay = w.layers[0]
    dl = dev_layer(lay)
    print("case append 64 users: T_hist", w.total, "T_new", int(adds.sum()), flush=True)
    kc, vc = gpu_cache(w, dl, w.offsets, w.x, w.ts)
    y, ko, vo = gpu_append(w, dl, w.offsets, w.ts, kc, vc, w.add_offsets, w.add_ts, w.x_new)
    yh = host(y)
    users = np.sort(np.argsort(w.lengths, kind="stable")[::5])
    hrows = np.concatenate([np.arange(w.offsets[u], w.offsets[u + 1]) for u in users])
    arows = np.concatenate([np.arange(w.add_offsets[u], w.add_offsets[u + 1]) for u in users])
    hoff, aoff = synth.offsets_of(w.lengths[users]), synth.offsets_of(adds[users])
    kv = oracle.layer_kv(w.x[hrows], lay, w.heads, w.d)
    ref, _ = oracle.layer_append(hoff, w.ts[hrows], aoff, w.add_ts[arows], lay, kv, w.x_new[arows], w.heads, w.d,
                                 w.n_max)
    branch_check("append 64 users (subset %s)" % users.tolist(), yh[arows], ref, w.x_new[arows])
