"""Helpers shared by the GPU parity tests: move seeded synthetic inputs to
the device and compare against the fp64 oracle."""
import numpy as np
import torch

BF16_TOL = 2e-2   # max|x - ref| / RMS(ref) for bf16 storage
F32_TOL = 1e-4    # same for fp32 storage


def dev():
    return torch.device("cuda:0")


def t_act(a, dtype):
    """Synthetic fp32 array (already bf16-representable when dtype is bf16) ->
    device tensor of the storage dtype."""
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev()).to(td)


def t_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev())


def t_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev())


def t_i64(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int64)).to(dev())


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    if rms == 0:
        return float(np.abs(got).max()) if got.size else 0.0
    return float(np.abs(got - ref).max() / rms)


def bf16_bound(ref):
    """Bound for an output stored in bf16: the kernel's arithmetic budget
    (BF16_TOL of the RMS) on top of the error that the ideal bf16 output --
    the fp64 reference rounded to nearest-even bf16 -- already has in this
    metric, rel_err(round_bf16(ref), ref).  For jagged attention outputs that
    rounding alone is 1-4 % of the RMS (their peaks are several times their
    RMS), so a flat 2e-2 would fail a correctly rounded result."""
    ref = np.asarray(ref, np.float64)
    return BF16_TOL + rel_err(round_bf16(ref), ref)


def round_bf16(a):
    """fp64 array -> the nearest bf16 values (ties to even), as fp64.  Each
    value is first taken to the nearest fp32 (exact for every input that is
    itself a bf16 or fp32 value), then to bf16."""
    t = torch.from_numpy(np.ascontiguousarray(a, np.float64)).to(torch.float32)
    return t.to(torch.bfloat16).to(torch.float64).numpy()


def sample_rows(offsets, n, rng):
    """Rows that cover every sequence's last (longest) row, its first row and
    random rows in between."""
    rows = set()
    for b in range(len(offsets) - 1):
        o, e = int(offsets[b]), int(offsets[b + 1])
        if e > o:
            rows.update([o, e - 1])
    T = int(offsets[-1])
    if T:
        rows.update(rng.choice(T, size=min(n, T), replace=False).tolist())
    return np.array(sorted(rows), np.int64)
