"""GPU parity of Stochastic Length sampling (hstu_sl_sample, the device
gather that builds the sampled jagged batch) through the C ABI against the
oracle: the sampled offsets and source rows bit for bit, the gathered rows
and times exactly."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import t_act, t_i32, t_i64

pytestmark = pytest.mark.gpu

hs = pytest.importorskip("hstu_sequential_transducer_amd")


def run(lengths, seed, alpha=1.6, distinct=0, with_x=True, u=None):
    L = np.asarray(lengths, np.int64)
    off = synth.offsets_of(L)
    T = int(off[-1])
    uu, keys = synth.sl_draws(seed, L, distinct)
    if u is not None:
        uu = np.full(len(L), u)
    ts = synth.timestamps(np.random.default_rng(seed + 1), L)
    x = np.random.default_rng(seed + 2).standard_normal((T, 512)).astype(np.float32)
    xd = t_act(x, "bf16") if with_x else None
    oo, oi, xo, to = hs.sl_sample(t_i32(off), T, t_i64(ts), alpha, torch.from_numpy(uu).to("cuda:0"),
                                  torch.from_numpy(keys.view(np.int32)).to("cuda:0"), xd)
    torch.cuda.synchronize()
    ref_off, ref_idx = oracle.sl_sample(off, alpha, uu, keys)
    got_off = oo.cpu().numpy()
    n_out = int(ref_off[-1])
    print("case sl lengths", list(L)[:8], "...", "kept", n_out, "of", T, flush=True)
    assert np.array_equal(got_off, ref_off)
    got_idx = oi.cpu().numpy()[:n_out]
    assert np.array_equal(got_idx, ref_idx)
    if with_x:
        assert torch.equal(xo[:n_out], xd[torch.from_numpy(ref_idx.astype(np.int64)).to("cuda:0")])
    assert np.array_equal(to.cpu().numpy()[:n_out], ts[ref_idx])
    return ref_off


def test_sl_small_ragged():
    run([0, 1, 5, 40, 1000, 3000, 2, 129], 111)


def test_sl_ties_and_extreme_draws():
    run([50, 300, 7, 1], 112, distinct=3)              # many equal keys: earlier positions first
    o = run([64, 9, 1000], 113, u=1.0)                   # u = 1 keeps everything
    assert list(np.diff(o)) == [64, 9, 1000]
    o = run([64, 9, 1000], 114, u=1e-300)                # a tiny u keeps one action each
    assert list(np.diff(o)) == [1, 1, 1]


def test_sl_headline_histories():
    """Eight full histories of 8192 actions (the pages' length 8192) and 64
    of 4096 (the layer workloads' n): the batches the attention path
    consumes, alpha = 1.6."""
    run(np.full(8, 8192), 115)
    run(np.full(64, 4096), 116, with_x=False)


def test_sl_histories_around_the_register_limit():
    """Histories of up to 8192 actions keep their keys in registers, longer
    ones re-read them every pass: lengths on both sides of the limit, with
    distinct keys and with heavy ties, and with everything kept."""
    run([8192, 8193, 20000, 1, 8191, 700], 117)
    run([8193, 8192, 12000, 3], 118, distinct=4)
    o = run([8192, 9000], 119, u=1.0)
    assert list(np.diff(o)) == [8192, 9000]
