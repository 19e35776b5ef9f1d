"""hstu_attn_fwd_noalloc (the forward with the library's static device
scratch array, for callers that cannot allocate) against hstu_attn_fwd (the
same kernels on a caller workspace), through the C ABI: bit-identical
outputs on two calls in a row, the second with a smaller batch, with and
without the LayerNorm gate."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import t_act, t_f32, t_i32, t_i64

pytestmark = pytest.mark.gpu

hs = pytest.importorskip("hstu_sequential_transducer_amd")


def _both(w, gate):
    T, F = w.total, w.heads * w.d
    dev_ = torch.device("cuda:0")
    q, k, v = (t_act(a, "bf16").reshape(T, w.heads, w.d) for a in (w.q, w.k, w.v))
    u = t_act(w.u, "bf16") if gate else None
    off, ts, rp, rt = t_i32(w.offsets), t_i64(w.ts), t_f32(w.rab_p), t_f32(w.rab_t)
    res = []
    for fn in (hs.attn_fwd, hs.attn_fwd_noalloc):
        out = torch.empty((T, F), dtype=torch.bfloat16, device=dev_)
        osv = torch.empty((T, F), dtype=torch.float32, device=dev_) if gate else None
        lst = torch.empty((T, 2), dtype=torch.float32, device=dev_) if gate else None
        fn(off, T, ts, q, k, v, rp, rt, w.n_max, u=u, eps=w.ln_eps, out=out, o_save=osv, ln_stats=lst)
        torch.cuda.synchronize()
        res.append((out, osv, lst))
    return res


@pytest.mark.parametrize("gate", [True, False])
def test_noalloc_matches_workspace_entry_point(gate):
    big = synth.attention_workload("noalloc-a", 81, np.array([700, 129, 1, 300, 2100]), heads=4, d=128,
                                   n_max=4096, epilogue=gate)
    small = synth.attention_workload("noalloc-b", 82, np.array([50, 3, 130]), heads=4, d=128, n_max=4096,
                                     epilogue=gate)
    for w in (big, small):
        print("case noalloc gate", gate, "lengths", list(w.lengths), flush=True)
        (a, ao, al), (b, bo, bl) = _both(w, gate)
        assert torch.equal(a, b)
        if gate:
            assert torch.equal(ao, bo) and torch.equal(al, bl)


def test_noalloc_gate_without_o_save_uses_staging_rows():
    """With u and no o_save the fp32 O rows are staged in the scratch array
    (this batch fits its limit)."""
    w = synth.attention_workload("noalloc-c", 83, np.array([200, 77]), heads=4, d=128, n_max=512, epilogue=True)
    T, F = w.total, w.heads * w.d
    q, k, v = (t_act(a, "bf16").reshape(T, w.heads, w.d) for a in (w.q, w.k, w.v))
    args = (t_i32(w.offsets), T, t_i64(w.ts), q, k, v, t_f32(w.rab_p), t_f32(w.rab_t), w.n_max)
    u = t_act(w.u, "bf16")
    a = hs.attn_fwd(*args, u=u, eps=w.ln_eps)
    a = a.clone()
    b = hs.attn_fwd_noalloc(*args, u=u, eps=w.ln_eps)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
