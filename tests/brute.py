"""Dense brute-force forms used to pin the loop oracle (test helper, fp64).

These are not the oracle: they evaluate the same definitions in a different
shape -- one padded dense matrix per sequence, an explicit lower-triangular
mask, a Toeplitz position-bias matrix built from an outer difference, time
buckets from Python's ``int.bit_length`` and SiLU from scipy's ``expit`` --
so that an indexing, sign or operand mistake in the loops shows up as a
disagreement.  Source of the definitions: paper review "Actions Speak Louder
than Words", section 3, Eq. 1-3.
"""
import numpy as np
import torch
from scipy.special import expit


def bucket_bitlen(dt: int) -> int:
    return min(127, (abs(int(dt)) + 1).bit_length() - 1)


def dense_attn(offsets, ts, q, k, v, rab_p, rab_t, n_max):
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    T, H, dqk = q.shape
    dv = v.shape[2]
    out = np.zeros((T, H * dv))
    for b in range(len(offsets) - 1):
        o, e = int(offsets[b]), int(offsets[b + 1])
        L = e - o
        if L == 0:
            continue
        ar = np.arange(L)
        rel = np.subtract.outer(ar, ar).T          # [i][j] = j - i
        pos = np.clip(rel, -n_max, n_max) + n_max
        mask = np.tril(np.ones((L, L), bool))      # j <= i
        if ts is not None:
            tt = [int(x) for x in ts[o:e]]
            bk = np.array([[bucket_bitlen(tt[i] - tt[j]) for j in range(L)] for i in range(L)])
        for h in range(H):
            S = q[o:e, h, :] @ k[o:e, h, :].T
            if rab_p is not None:
                S = S + np.asarray(rab_p, np.float64)[h][pos]
            if rab_t is not None and ts is not None:
                S = S + np.asarray(rab_t, np.float64)[h][bk]
            P = np.where(mask, S * expit(S), 0.0)
            out[o:e, h * dv:(h + 1) * dv] = P @ v[o:e, h, :] / n_max
    return out


def dense_ln_gate(O, U, eps):
    Ot = torch.from_numpy(np.asarray(O, np.float64))
    xh = torch.nn.functional.layer_norm(Ot, (Ot.shape[-1],), eps=eps)
    return (xh * torch.from_numpy(np.asarray(U, np.float64))).numpy()


def dense_layer(offsets, ts, x, layer, H, d, n_max, phi1=0, eps=1e-5):
    X = torch.from_numpy(np.asarray(x, np.float64))
    Z = torch.nn.functional.linear(X, torch.from_numpy(np.asarray(layer.w1, np.float64)),
                                   torch.from_numpy(np.asarray(layer.b1, np.float64)))
    A = torch.nn.functional.silu(Z) if phi1 == 0 else torch.relu(Z)
    HD = H * d
    T = X.shape[0]
    U, V, Q, K = (A[:, i * HD:(i + 1) * HD].numpy() for i in range(4))
    O = dense_attn(offsets, ts, Q.reshape(T, H, d), K.reshape(T, H, d), V.reshape(T, H, d), layer.rab_p,
                   layer.rab_t, n_max)
    G = dense_ln_gate(O, U, eps)
    Y = X + torch.nn.functional.linear(torch.from_numpy(G), torch.from_numpy(np.asarray(layer.w2, np.float64)),
                                       torch.from_numpy(np.asarray(layer.b2, np.float64)))
    return Y.numpy(), K.reshape(T, H, d), V.reshape(T, H, d)
