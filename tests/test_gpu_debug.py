"""Device-side data checks through the C ABI: with HSTU_DEBUG=1 a call
synchronises its stream and reports a batch whose offsets fail the
launcher's check (offsets[0] != 0, decreasing, offsets[B] != total) as
HSTU_ERR_ARG; the attention entry points then leave their outputs
untouched."""
import ctypes
import os

import numpy as np
import pytest
import torch

import synth
from gpu_util import t_act, t_f32, t_i32, t_i64

pytestmark = pytest.mark.gpu

hs = pytest.importorskip("hstu_sequential_transducer_amd")
from hstu_sequential_transducer_amd import binding as bd  # noqa: E402


@pytest.fixture
def debug_env():
    old = os.environ.get("HSTU_DEBUG")
    os.environ["HSTU_DEBUG"] = "1"
    yield
    if old is None:
        del os.environ["HSTU_DEBUG"]
    else:
        os.environ["HSTU_DEBUG"] = old


SENTINEL = 7.0


def _case():
    w = synth.attention_workload("dbg", 71, np.array([50, 30, 80]), heads=4, d=128, n_max=128, epilogue=True,
                                 with_grad=True)
    T, F = w.total, w.heads * w.d
    dev_ = torch.device("cuda:0")
    t = dict(q=t_act(w.q, "bf16").reshape(T, 4, 128), k=t_act(w.k, "bf16").reshape(T, 4, 128),
             v=t_act(w.v, "bf16").reshape(T, 4, 128), u=t_act(w.u, "bf16"), dg=t_act(w.dg, "bf16"),
             ts=t_i64(w.ts), rp=t_f32(w.rab_p), rt=t_f32(w.rab_t))
    fill = lambda shape, dt: torch.full(shape, SENTINEL, dtype=dt, device=dev_)
    return w, t, fill


def _fwd_raw(w, t, off, out, osv, lst):
    lib = hs.load_library()
    T, H, d = w.total, w.heads, w.d
    jag = bd._jagged(off, t["ts"], w.n_max, T)
    dims = bd.Dims(bd.HSTU_BF16, H, d, d, w.ln_eps)
    ws = torch.empty(bd.workspace_size(bd.OP_ATTN_FWD, jag, dims), dtype=torch.uint8, device=out.device)
    bias = bd._bias(t["rp"], t["rt"])
    return lib.hstu_attn_fwd(ctypes.byref(jag), ctypes.byref(dims), ctypes.byref(bias), bd._rowmat(t["q"], H * d),
                             bd._rowmat(t["k"], H * d), bd._rowmat(t["v"], H * d), bd._rowmat(t["u"], H * d),
                             bd._rowmat(out, H * d, bd.Mat), osv.data_ptr(), lst.data_ptr(), ws.data_ptr(), ws.numel(),
                             bd._stream(out.device))


def _bwd_raw(w, t, off, osv, lst, outs):
    lib = hs.load_library()
    T, H, d = w.total, w.heads, w.d
    jag = bd._jagged(off, t["ts"], w.n_max, T)
    dims = bd.Dims(bd.HSTU_BF16, H, d, d, w.ln_eps)
    ws = torch.empty(bd.workspace_size(bd.OP_ATTN_BWD, jag, dims), dtype=torch.uint8, device=osv.device)
    bias = bd._bias(t["rp"], t["rt"])
    m = lambda x: bd._rowmat(x, H * d, bd.Mat)
    return lib.hstu_attn_bwd(ctypes.byref(jag), ctypes.byref(dims), ctypes.byref(bias), bd._rowmat(t["q"], H * d),
                             bd._rowmat(t["k"], H * d), bd._rowmat(t["v"], H * d), bd._rowmat(t["u"], H * d),
                             osv.data_ptr(), lst.data_ptr(), bd._rowmat(t["dg"], H * d), m(outs["dq"]), m(outs["dk"]),
                             m(outs["dv"]), m(outs["du"]), outs["drab_p"].data_ptr(), outs["drab_t"].data_ptr(),
                             ws.data_ptr(), ws.numel(), bd._stream(osv.device))


@pytest.mark.parametrize("bad", ["decreasing", "first_not_zero", "last_not_total"])
def test_debug_bad_offsets_reported_outputs_untouched(debug_env, bad):
    w, t, fill = _case()
    T, F = w.total, w.heads * w.d
    good = w.offsets.astype(np.int32)
    offs = {"decreasing": np.array([0, 50, 30, 160], np.int32),
            "first_not_zero": np.array([4, 50, 80, 160], np.int32),
            "last_not_total": np.array([0, 50, 80, 150], np.int32)}[bad]
    print("case debug", bad, "offsets", offs.tolist(), flush=True)
    off = t_i32(offs)
    out, osv, lst = fill((T, F), torch.bfloat16), fill((T, F), torch.float32), fill((T, 2), torch.float32)
    st = _fwd_raw(w, t, off, out, osv, lst)
    assert st == bd.HSTU_ERR_ARG, (st, hs.last_error())
    assert "offsets" in hs.last_error()
    torch.cuda.synchronize()
    for x in (out, osv, lst):
        assert bool((x.float() == SENTINEL).all())
    # the forward with valid offsets, then the backward with the bad ones
    assert _fwd_raw(w, t, t_i32(good), out, osv, lst) == bd.HSTU_OK, hs.last_error()
    outs = dict(dq=fill((T, 4, 128), torch.bfloat16), dk=fill((T, 4, 128), torch.bfloat16),
                dv=fill((T, 4, 128), torch.bfloat16), du=fill((T, F), torch.bfloat16),
                drab_p=fill(tuple(w.rab_p.shape), torch.float32), drab_t=fill(tuple(w.rab_t.shape), torch.float32))
    st = _bwd_raw(w, t, off, osv, lst, outs)
    assert st == bd.HSTU_ERR_ARG, (st, hs.last_error())
    torch.cuda.synchronize()
    for n, x in outs.items():
        assert bool((x.float() == SENTINEL).all()), n
    # and the same call with valid offsets succeeds and writes them
    assert _bwd_raw(w, t, t_i32(good), osv, lst, outs) == bd.HSTU_OK, hs.last_error()
    torch.cuda.synchronize()
    assert not bool((outs["dq"].float() == SENTINEL).all())


def test_debug_mfalcon_history_total_mismatch(debug_env):
    """M-FALCON's launcher checks hist offsets[U] against the history total
    (the key splits are sized from it)."""
    w = synth.mfalcon_workload("dbg-mf", 72, np.array([40, 60]), cands_per_user=3, n_max=128, n_layers=1)
    T, H, d = w.total, w.heads, w.d
    dev_ = torch.device("cuda:0")
    lay = dict(w1=t_act(w.layers[0].w1, "bf16"), b1=t_f32(w.layers[0].b1), w2=t_act(w.layers[0].w2, "bf16"),
               b2=t_f32(w.layers[0].b2), rab_p=t_f32(w.layers[0].rab_p), rab_t=t_f32(w.layers[0].rab_t), phi1=0)
    kc = torch.zeros((T + 8, H * d), dtype=torch.bfloat16, device=dev_)
    vc = torch.zeros_like(kc)
    xc = t_act(w.x_cand, "bf16")
    M = xc.shape[0]
    bad = t_i32(np.array([0, 40, 90], np.int32))  # offsets[U] = 90, total says 100
    with pytest.raises(hs.HstuError) as e:
        hs.mfalcon_score(bad, T, t_i64(w.ts), [lay], [kc], [vc], t_i32(w.cand_offsets), M, t_i64(w.cand_ts), xc, 2,
                         H, d, w.n_max)
    assert e.value.status == bd.HSTU_ERR_ARG
    assert "offsets" in str(e.value)
    y = hs.mfalcon_score(t_i32(w.offsets), T, t_i64(w.ts), [lay], [kc], [vc], t_i32(w.cand_offsets), M,
                         t_i64(w.cand_ts), xc, 2, H, d, w.n_max)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all())
