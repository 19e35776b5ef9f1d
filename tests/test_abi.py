"""The C ABI library loads and exports every symbol include/hstu.h declares,
and host-side argument validation rejects bad calls before any device work
(no GPU needed: every call below returns before touching HIP)."""
import ctypes
import os
import re

import pytest

import hstu_sequential_transducer_amd as hs
from hstu_sequential_transducer_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hstu.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)
    skip = {"if", "sizeof", "defined"}
    return sorted({n for n in names if n not in skip and (n.startswith("hstu_") or n.startswith("mfalcon_"))})


def test_library_exports_every_declared_symbol():
    lib = hs.load_library()
    decl = declared_functions()
    assert set(decl) == set(bd.EXPORTED), decl
    for name in decl:
        assert hasattr(lib, name), name


def test_abi_version_matches_header():
    m = re.search(r"#define HSTU_ABI_VERSION (\d+)", open(HEADER).read())
    assert hs.abi_version() == int(m.group(1))


def _dims(dtype=bd.HSTU_BF16, H=4, d=128, eps=1e-5):
    return bd.Dims(dtype, H, d, d, eps)


def _jag(B=2, T=10, n=8, off=1, ts=None):
    return bd.Jagged(B, T, n, off, ts)


def _call_fwd(jag, dims, ws=None, ws_bytes=0, q=256, ldq=512, out=1024, k=512, ldk=512, o_save=None):
    """hstu_attn_fwd with made-up device addresses (never dereferenced: every
    case below fails validation before anything is enqueued)."""
    lib = hs.load_library()
    bias = bd.Bias(None, 0, None, 0)
    m = lambda p, ld: bd.CMat(p, ld)
    return lib.hstu_attn_fwd(ctypes.byref(jag) if jag is not None else None, ctypes.byref(dims), ctypes.byref(bias),
                             m(q, ldq), m(k, ldk), m(768, 512), m(None, 0), bd.Mat(out, 512), o_save, None, ws,
                             ws_bytes, None)


def test_validation_errors_are_reported():
    assert _call_fwd(None, _dims()) == bd.HSTU_ERR_ARG
    assert "NULL" in hs.last_error()
    assert _call_fwd(_jag(B=0), _dims()) == bd.HSTU_ERR_ARG
    assert _call_fwd(_jag(n=0), _dims()) == bd.HSTU_ERR_ARG
    assert _call_fwd(_jag(), _dims(d=48)) == bd.HSTU_ERR_UNSUPPORTED
    assert _call_fwd(_jag(), _dims(d=256)) == bd.HSTU_ERR_UNSUPPORTED
    assert _call_fwd(_jag(), _dims(d=64), ldq=256, ldk=256) == bd.HSTU_ERR_WORKSPACE  # d = 64 passes validation
    assert _call_fwd(_jag(), _dims(dtype=bd.HSTU_F32, d=24)) == bd.HSTU_ERR_UNSUPPORTED
    assert _call_fwd(_jag(), _dims(eps=0.0)) == bd.HSTU_ERR_ARG
    assert _call_fwd(_jag(), _dims(), q=None) == bd.HSTU_ERR_ARG
    assert _call_fwd(_jag(), _dims(), ldq=100) == bd.HSTU_ERR_ARG
    assert "ld" in hs.last_error()
    assert _call_fwd(_jag(), _dims(), ldq=1 << 24) == bd.HSTU_ERR_UNSUPPORTED
    assert "2^24" in hs.last_error()
    assert _call_fwd(_jag(), _dims(), ws=None) == bd.HSTU_ERR_WORKSPACE
    assert _call_fwd(_jag(), _dims(), ws=256 * 3 + 4, ws_bytes=1 << 30) == bd.HSTU_ERR_WORKSPACE
    assert _call_fwd(_jag(), _dims(), ws=256 * 4, ws_bytes=16) == bd.HSTU_ERR_WORKSPACE
    assert "too small" in hs.last_error()


def test_bf16_views_must_be_16_byte_aligned():
    """bf16 Q/K/V/U/outputs are moved with 16-byte accesses: a base that is
    not 16-byte aligned, or a token stride that is not a multiple of 8
    elements, is rejected before any launch; so is an fp32 o_save that is not
    16-byte aligned."""
    assert _call_fwd(_jag(), _dims(), q=256 + 4) == bd.HSTU_ERR_ARG
    assert "16-byte" in hs.last_error() and "q" in hs.last_error()
    assert _call_fwd(_jag(), _dims(), k=512 + 8) == bd.HSTU_ERR_ARG
    assert _call_fwd(_jag(), _dims(), ldk=516) == bd.HSTU_ERR_ARG
    assert "multiple of 8" in hs.last_error()
    assert _call_fwd(_jag(), _dims(), out=1024 + 2) == bd.HSTU_ERR_ARG
    assert _call_fwd(_jag(), _dims(), o_save=2048 + 4) == bd.HSTU_ERR_ARG
    assert "o_save" in hs.last_error()
    # fp32 views keep 4-byte alignment (the fp32 kernel reads them one by one)
    assert _call_fwd(_jag(), _dims(dtype=bd.HSTU_F32, d=32), q=256 + 4, ldq=128, ldk=128, k=512) == bd.HSTU_ERR_WORKSPACE


def _call_bwd(dq=1280, lddq=512):
    lib = hs.load_library()
    bias = bd.Bias(None, 0, None, 0)
    c = lambda p: bd.CMat(p, 512)
    return lib.hstu_attn_bwd(ctypes.byref(_jag()), ctypes.byref(_dims()), ctypes.byref(bias), c(256), c(512), c(768),
                             c(None), None, None, c(1024), bd.Mat(dq, lddq), bd.Mat(1536, 512), bd.Mat(1792, 512),
                             bd.Mat(None, 0), None, None, None, 0, None)


def test_bwd_views_checked_before_launch():
    lib = hs.load_library()
    call = lambda d: lib.hstu_attn_bwd(ctypes.byref(_jag()), ctypes.byref(_dims(d=d)), None,
                                       *(bd.CMat(256, 512),) * 3, bd.CMat(None, 0), None, None, bd.CMat(1024, 512),
                                       *(bd.Mat(1280, 512),) * 3, bd.Mat(None, 0), None, None, None, 0, None)
    assert call(48) == bd.HSTU_ERR_UNSUPPORTED
    assert "{32, 64, 128}" in hs.last_error()
    assert call(64) == bd.HSTU_ERR_WORKSPACE  # d = 64 passes validation
    assert _call_bwd(dq=1280 + 8) == bd.HSTU_ERR_ARG
    assert "dq" in hs.last_error()
    assert _call_bwd(lddq=520 + 4) == bd.HSTU_ERR_ARG
    assert _call_bwd() == bd.HSTU_ERR_WORKSPACE


def test_workspace_size_grows_with_tokens():
    lib = hs.load_library()
    d = _dims()
    small = lib.hstu_workspace_size(bd.OP_ATTN_FWD, ctypes.byref(_jag(T=100)), ctypes.byref(d), 0, 0)
    big = lib.hstu_workspace_size(bd.OP_ATTN_FWD, ctypes.byref(_jag(T=100000)), ctypes.byref(d), 0, 0)
    assert 0 < small < big
    assert big % 256 == 0
    assert lib.hstu_workspace_size(bd.OP_ATTN_FWD, ctypes.byref(_jag(B=0)), ctypes.byref(d), 0, 0) == 0


def _call_layer_bwd(dims, D=512, x=256, dy=512, dx=768, dw1=1024, dw2=1280, db1=None, w1=1536, ws=None, ws_bytes=0):
    lib = hs.load_library()
    lay = bd.Layer(w1, None, 1792, None, bd.Bias(None, 0, None, 0), bd.HSTU_ACT_SILU)
    return lib.hstu_layer_bwd(ctypes.byref(_jag()), ctypes.byref(dims), D, ctypes.byref(lay), bd.CMat(x, D),
                              bd.CMat(dy, D), bd.Mat(dx, D), dw1, db1, dw2, None, None, None, ws, ws_bytes, None)


def test_layer_bwd_validation():
    """hstu_layer_bwd rejects what it does not take before enqueuing
    anything (the pointers here are never dereferenced)."""
    assert _call_layer_bwd(_dims(dtype=bd.HSTU_F32, d=32)) == bd.HSTU_ERR_UNSUPPORTED
    assert _call_layer_bwd(_dims(d=64)) == bd.HSTU_ERR_UNSUPPORTED  # the layer keeps d = 128
    assert "d = 128" in hs.last_error()
    assert _call_layer_bwd(_dims(), D=70) == bd.HSTU_ERR_UNSUPPORTED
    assert "multiple of 8" in hs.last_error()
    assert _call_layer_bwd(_dims(), dx=256) == bd.HSTU_ERR_ARG
    assert "alias" in hs.last_error()
    assert _call_layer_bwd(_dims(), dw1=None) == bd.HSTU_ERR_ARG
    assert _call_layer_bwd(_dims(), db1=1024 + 4) == bd.HSTU_ERR_ARG
    assert "16-byte" in hs.last_error()
    assert _call_layer_bwd(_dims(), w1=None) == bd.HSTU_ERR_ARG
    assert _call_layer_bwd(_dims()) == bd.HSTU_ERR_WORKSPACE


def test_layer_bwd_workspace_size():
    lib = hs.load_library()
    d = _dims()
    small = lib.hstu_workspace_size(bd.OP_LAYER_BWD, ctypes.byref(_jag(T=100)), ctypes.byref(d), 512, 0)
    big = lib.hstu_workspace_size(bd.OP_LAYER_BWD, ctypes.byref(_jag(T=100000)), ctypes.byref(d), 512, 0)
    attn = lib.hstu_workspace_size(bd.OP_ATTN_BWD, ctypes.byref(_jag(T=100000)), ctypes.byref(d), 0, 0)
    assert 0 < small < big and big > attn and big % 256 == 0
    assert lib.hstu_workspace_size(bd.OP_LAYER_BWD, ctypes.byref(_jag(T=100)), ctypes.byref(d), 0, 0) == 0


def test_noalloc_rejects_batches_beyond_its_scratch_limit():
    """hstu_attn_fwd_noalloc validates like hstu_attn_fwd and refuses a batch
    whose scratch would exceed HSTU_NOALLOC_SCRATCH_BYTES before touching the
    device (the pointers are never dereferenced)."""
    lib = hs.load_library()
    limit = int(re.search(r"#define HSTU_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
                .group(1)) << 20
    assert limit == 16 << 20
    bias = bd.Bias(None, 0, None, 0)
    m = lambda p, ld=512: bd.CMat(p, ld)
    call = lambda T, u=None, o_save=None: lib.hstu_attn_fwd_noalloc(
        ctypes.byref(_jag(T=T)), ctypes.byref(_dims()), ctypes.byref(bias), m(256), m(512), m(768), m(u),
        bd.Mat(1024, 512), o_save, None, None)
    assert call(2_000_000) == bd.HSTU_ERR_WORKSPACE      # 12 bytes of relative time per token alone
    assert "limit" in hs.last_error()
    assert call(20_000, u=1280) == bd.HSTU_ERR_WORKSPACE  # fp32 O staging rows for the gate
    assert "o_save" in hs.last_error()
    assert lib.hstu_attn_fwd_noalloc(ctypes.byref(_jag()), ctypes.byref(_dims(d=48)), ctypes.byref(bias), m(256),
                                     m(512), m(768), m(None), bd.Mat(1024, 512), None, None,
                                     None) == bd.HSTU_ERR_UNSUPPORTED
