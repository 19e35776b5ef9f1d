"""Seeded synthetic inputs for the HSTU attention path.

This module is shared by the CPU oracle (``oracle/``), the tests and the
benchmark.  It holds no arithmetic of the method itself: it only draws random
numbers, rounds them to the storage dtype and lays them out.  The workloads
take their shapes and distributions from the pages on HSTU / Generative
Recommenders (review of "Actions Speak Louder than Words", section 3: core
formulas and Stochastic Length): jagged sequences up to N_max = 8192, H = 4
heads of d = 128, integer timestamps, small N(0, 0.02) tables and weights.

Draw order inside one workload is fixed (a change of it changes every input):
lengths -> timestamp gaps (per sequence) -> weights and tables in layer order
(W1, b1, W2, b2, rab_p, rab_t) -> activations (X, or Q, K, V, U) -> upstream
gradient -> candidate time gaps -> candidates.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np
import torch

EPOCH = 1_700_000_000  # seconds; a realistic absolute origin so times need int64
TIME_GAP_MEAN = 60.0   # mean gap between two actions of one user (seconds)
TABLE_STD = 0.02       # std of weights and rab tables ("N(0, 0.02)")
RAB_T_BUCKETS = 128


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round an fp32 array to the nearest bf16 value (ties to even) and return
    it as fp32, so that every consumer sees exactly the stored values."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def stochastic_lengths(rng: np.random.Generator, batch: int, n: int, alpha: float) -> np.ndarray:
    """Sequence lengths from the Stochastic Length law of the paper review
    "Actions Speak Louder than Words" (section 3, Stochastic Length):
    L = min(n, ceil(n * u**(1/alpha))), u ~ U(0, 1).  A draw of u = 0 would
    give L = 0; it is clamped to 1."""
    u = rng.random(batch)
    L = np.minimum(n, np.ceil(n * u ** (1.0 / alpha))).astype(np.int64)
    return np.maximum(L, 1)


def timestamps(rng: np.random.Generator, lengths: np.ndarray) -> np.ndarray:
    """Per sequence: t_k = EPOCH + floor(sum_{r<=k} g_r), g ~ Exp(mean 60 s).
    Non-decreasing inside each sequence, int64 seconds."""
    out = []
    for L in lengths:
        g = rng.exponential(TIME_GAP_MEAN, size=int(L))
        out.append(EPOCH + np.floor(np.cumsum(g)).astype(np.int64))
    return np.concatenate(out) if out else np.zeros(0, np.int64)


def offsets_of(lengths: np.ndarray) -> np.ndarray:
    off = np.zeros(len(lengths) + 1, np.int32)
    off[1:] = np.cumsum(lengths)
    return off


@dataclasses.dataclass
class Layer:
    """One HSTU layer's parameters, fp32 arrays (bf16-representable when the
    workload is bf16).  Linear weights use the [out][in] layout: y = x W^T + b.
    w1: [4*H*d][D] with output column blocks U | V | Q | K (head-major inside),
    w2: [D][H*d]; rab_p: [H][2*N_max+1]; rab_t: [H][128]."""
    w1: np.ndarray
    b1: np.ndarray
    w2: np.ndarray
    b2: np.ndarray
    rab_p: np.ndarray
    rab_t: np.ndarray


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str                  # "f32" or "bf16": storage dtype of activations
    heads: int
    d: int                      # d_qk == d_v
    n_max: int
    lengths: np.ndarray         # int64 [B]
    offsets: np.ndarray         # int32 [B+1]
    ts: np.ndarray              # int64 [T]
    rab_p: np.ndarray           # fp32 [H][2N+1]
    rab_t: np.ndarray           # fp32 [H][128]
    d_model: int = 0
    layers: List[Layer] = dataclasses.field(default_factory=list)
    x: Optional[np.ndarray] = None   # [T][D]
    q: Optional[np.ndarray] = None   # [T][H][d]
    k: Optional[np.ndarray] = None
    v: Optional[np.ndarray] = None
    u: Optional[np.ndarray] = None   # [T][H*d]
    dg: Optional[np.ndarray] = None  # [T][H*d] upstream gradient at G
    dy: Optional[np.ndarray] = None  # [T][D] upstream gradient at the layer output Y
    epilogue: bool = True
    ln_eps: float = 1e-5
    # M-FALCON
    cand_offsets: Optional[np.ndarray] = None   # int32 [U+1]
    cand_ts: Optional[np.ndarray] = None        # int64 [U]
    x_cand: Optional[np.ndarray] = None         # [M][D]
    b_m: int = 0

    @property
    def batch(self) -> int:
        return len(self.lengths)

    @property
    def total(self) -> int:
        return int(self.offsets[-1])


def _normal(rng, shape, std, dtype):
    a = (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)
    return round_bf16(a) if dtype == "bf16" else a


def _layer(rng, D, H, d, N, dtype, rab_std=TABLE_STD):
    w1 = _normal(rng, (4 * H * d, D), TABLE_STD, dtype)
    b1 = np.zeros(4 * H * d, np.float32)
    w2 = _normal(rng, (D, H * d), TABLE_STD, dtype)
    b2 = np.zeros(D, np.float32)
    rab_p = _normal(rng, (H, 2 * N + 1), rab_std, "f32")
    rab_t = _normal(rng, (H, RAB_T_BUCKETS), rab_std, "f32")
    return Layer(w1, b1, w2, b2, rab_p, rab_t)


def attention_workload(name: str, seed: int, lengths: Optional[np.ndarray], *, heads: int, d: int,
                       n_max: int, dtype: str = "bf16", epilogue: bool = True,
                       with_grad: bool = False, sl: Optional[tuple] = None,
                       act_std: Optional[float] = None, batch: int = 0,
                       uniform_len: Optional[tuple] = None) -> Workload:
    """Attention-only workload: Q, K, V, U ~ N(0,1)/sqrt(d) (or act_std),
    tables ~ N(0, 0.02), timestamps as above, dG ~ N(0, 1)."""
    rng = np.random.default_rng(seed)
    if lengths is None:
        if sl is not None:
            lengths = stochastic_lengths(rng, batch, sl[0], sl[1])
        else:
            lo, hi = uniform_len
            lengths = rng.integers(lo, hi + 1, size=batch).astype(np.int64)
    lengths = np.asarray(lengths, np.int64)
    ts = timestamps(rng, lengths)
    H = heads
    rab_p = _normal(rng, (H, 2 * n_max + 1), TABLE_STD, "f32")
    rab_t = _normal(rng, (H, RAB_T_BUCKETS), TABLE_STD, "f32")
    T = int(lengths.sum())
    std = act_std if act_std is not None else 1.0 / math.sqrt(d)
    q = _normal(rng, (T, H, d), std, dtype)
    k = _normal(rng, (T, H, d), std, dtype)
    v = _normal(rng, (T, H, d), std, dtype)
    u = _normal(rng, (T, H * d), std, dtype)
    dg = _normal(rng, (T, H * d), 1.0, dtype) if with_grad else None
    return Workload(name=name, dtype=dtype, heads=H, d=d, n_max=n_max, lengths=lengths,
                    offsets=offsets_of(lengths), ts=ts, rab_p=rab_p, rab_t=rab_t,
                    q=q, k=k, v=v, u=u, dg=dg, epilogue=epilogue)


def layer_workload(name: str, seed: int, lengths: Optional[np.ndarray], *, d_model: int, heads: int,
                   d: int, n_max: int, dtype: str, n_layers: int = 1, with_grad: bool = False,
                   sl: Optional[tuple] = None, batch: int = 0) -> Workload:
    rng = np.random.default_rng(seed)
    if lengths is None:
        lengths = stochastic_lengths(rng, batch, sl[0], sl[1])
    lengths = np.asarray(lengths, np.int64)
    ts = timestamps(rng, lengths)
    layers = [_layer(rng, d_model, heads, d, n_max, dtype) for _ in range(n_layers)]
    T = int(lengths.sum())
    x = _normal(rng, (T, d_model), 1.0, dtype)
    dg = _normal(rng, (T, heads * d), 1.0, dtype) if with_grad else None
    dy = _normal(rng, (T, d_model), 1.0, dtype) if with_grad else None
    return Workload(name=name, dtype=dtype, heads=heads, d=d, n_max=n_max, lengths=lengths,
                    offsets=offsets_of(lengths), ts=ts, rab_p=layers[0].rab_p, rab_t=layers[0].rab_t,
                    d_model=d_model, layers=layers, x=x, dg=dg, dy=dy)


def mfalcon_workload(name: str, seed: int, hist_lengths: Optional[np.ndarray], *, cands_per_user: int,
                     d_model: int = 512, heads: int = 4, d: int = 128, n_max: int = 4096,
                     n_layers: int = 2, b_m: int = 256, dtype: str = "bf16",
                     sl: Optional[tuple] = None, users: int = 0) -> Workload:
    """M-FALCON ranking workload: per-user history X_h ~ N(0,1) that builds the
    per-layer K/V cache, and cands_per_user candidate tokens ~ N(0,1) per user.
    A candidate's time is the user's last history time + floor(Exp(60))."""
    rng = np.random.default_rng(seed)
    if hist_lengths is None:
        hist_lengths = stochastic_lengths(rng, users, sl[0], sl[1])
    hist_lengths = np.asarray(hist_lengths, np.int64)
    ts = timestamps(rng, hist_lengths)
    layers = [_layer(rng, d_model, heads, d, n_max, dtype) for _ in range(n_layers)]
    T = int(hist_lengths.sum())
    x = _normal(rng, (T, d_model), 1.0, dtype)
    offs = offsets_of(hist_lengths)
    U = len(hist_lengths)
    gaps = np.floor(rng.exponential(TIME_GAP_MEAN, size=U)).astype(np.int64)
    last = np.array([ts[offs[i + 1] - 1] if hist_lengths[i] > 0 else EPOCH for i in range(U)], np.int64)
    cand_ts = last + gaps
    cand_counts = np.full(U, cands_per_user, np.int64)
    M = int(cand_counts.sum())
    x_cand = _normal(rng, (M, d_model), 1.0, dtype)
    return Workload(name=name, dtype=dtype, heads=heads, d=d, n_max=n_max, lengths=hist_lengths,
                    offsets=offs, ts=ts, rab_p=layers[0].rab_p, rab_t=layers[0].rab_t,
                    d_model=d_model, layers=layers, x=x, cand_offsets=offsets_of(cand_counts),
                    cand_ts=cand_ts, x_cand=x_cand, b_m=b_m)


# ---------------------------------------------------------------------------
# The five named workloads.  Seeds: workload i uses seed i.

def tiny_layer_f32() -> Workload:
    """Tiny fp32 single layer: B=4, lengths {17, 64, 33, 5}, N_max=64, D=64,
    H=2, d=32, seed 0."""
    return layer_workload("tiny-layer-f32", 0, np.array([17, 64, 33, 5]), d_model=64, heads=2, d=32,
                          n_max=64, dtype="f32")


def attn_fwd_1k(seed: int = 1) -> Workload:
    """bf16 attention forward: B=32, lengths ~ U{64..1024}, N_max=1024, H=4,
    d=128, no epilogue."""
    return attention_workload("attn-fwd-B32-N1024", seed, None, heads=4, d=128, n_max=1024,
                              epilogue=False, batch=32, uniform_len=(64, 1024))


def attn_8k(seed: int = 2, with_grad: bool = True) -> Workload:
    """bf16 attention at N_max=8192: B=8, Stochastic-Length lengths (alpha 1.6,
    n=8192), H=4, d=128, LayerNorm(AV)*U epilogue; dG ~ N(0,1) for the
    backward."""
    return attention_workload("attn-8k-B8-SL1.6", seed, None, heads=4, d=128, n_max=8192,
                              epilogue=True, with_grad=with_grad, batch=8, sl=(8192, 1.6))


def layer_train_4k(seed: int = 3) -> Workload:
    """bf16 layer train step: B=16, SL(alpha 1.6, n=4096), N_max=4096, D=512,
    H=4, d=128, upstream gradients ~ N(0,1) at G (dg) and at Y (dy)."""
    return layer_workload("layer-train-B16-N4096", seed, None, d_model=512, heads=4, d=128, n_max=4096,
                          dtype="bf16", with_grad=True, sl=(4096, 1.6), batch=16)


def mfalcon_1user(seed: int = 4) -> Workload:
    """M-FALCON: one user, history 4096, 2 layers, m=1024 candidates, b_m=256."""
    return mfalcon_workload("mfalcon-1user-n4096-m1024", seed, np.array([4096]), cands_per_user=1024)


def mfalcon_64users(seed: int = 4) -> Workload:
    """M-FALCON: 64 users, histories SL(alpha 1.6, n=4096), m=1024 each."""
    # Drawn from its own stream so the 1-user workload is unchanged.
    return mfalcon_workload("mfalcon-64users-SL-m1024", seed * 1000 + 64, None, cands_per_user=1024,
                            sl=(4096, 1.6), users=64)


def append_workload(name: str, seed: int, hist_lengths, add_lengths, *, d_model: int = 512, heads: int = 4,
                    d: int = 128, n_max: int = 4096, n_layers: int = 1, dtype: str = "bf16") -> Workload:
    """New actions appended to cached user histories: per user a history of
    hist_lengths[u] actions (x, ts, which build the cache) and add_lengths[u]
    new actions (x_new, ts_new) whose times continue the user's history
    (last history time + cumulative Exp(60) gaps).  The new actions are kept
    in fields of their own: add_offsets, add_ts, x_new."""
    rng = np.random.default_rng(seed)
    hl = np.asarray(hist_lengths, np.int64)
    al = np.asarray(add_lengths, np.int64)
    ts = timestamps(rng, hl)
    offs = offsets_of(hl)
    add_ts = []
    for u in range(len(hl)):
        last = ts[offs[u + 1] - 1] if hl[u] > 0 else EPOCH
        g = rng.exponential(TIME_GAP_MEAN, size=int(al[u]))
        add_ts.append(last + np.floor(np.cumsum(g)).astype(np.int64))
    add_ts = np.concatenate(add_ts) if len(add_ts) else np.zeros(0, np.int64)
    layers = [_layer(rng, d_model, heads, d, n_max, dtype) for _ in range(n_layers)]
    x = _normal(rng, (int(hl.sum()), d_model), 1.0, dtype)
    x_new = _normal(rng, (int(al.sum()), d_model), 1.0, dtype)
    w = Workload(name=name, dtype=dtype, heads=heads, d=d, n_max=n_max, lengths=hl, offsets=offs, ts=ts,
                 rab_p=layers[0].rab_p, rab_t=layers[0].rab_t, d_model=d_model, layers=layers, x=x)
    w.add_offsets = offsets_of(al)
    w.add_ts = add_ts
    w.x_new = x_new
    return w


def sl_draws(seed: int, lengths, distinct_keys: int = 0):
    """The random numbers of Stochastic Length sampling for sequences of the
    given full lengths: u ~ U(0, 1) per sequence (fp64) and a uint32 key per
    action (uniform; or uniform over `distinct_keys` values, to force ties)."""
    rng = np.random.default_rng(seed)
    L = np.asarray(lengths, np.int64)
    u = rng.random(len(L))
    hi = distinct_keys if distinct_keys > 0 else 2 ** 32
    keys = rng.integers(0, hi, size=int(L.sum()), dtype=np.uint64).astype(np.uint32)
    return u, keys
