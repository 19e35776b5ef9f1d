"""hstu_sequential_transducer_amd -- HSTU pointwise aggregated attention for
AMD Instinct MI355X (gfx950): hand-written HIP kernels behind the C ABI of
include/hstu.h (libhstu.so), with a thin ctypes binding.

The method is the HSTU layer of Generative Recommenders (paper review
"Actions Speak Louder than Words", arXiv 2402.17152, section 3).
"""
from .binding import (HSTU_ACT_RELU, HSTU_ACT_SILU, HSTU_BF16, HSTU_F32, HstuError, LIB_PATH, abi_version,
                      attn_bwd, attn_fwd, attn_fwd_noalloc, last_error, layer_append, layer_bwd, layer_fwd, load_library, mfalcon_score,
                      profile_collect, profile_enable, sl_sample, softmax_attn_fwd)

__all__ = ["attn_fwd", "attn_fwd_noalloc", "attn_bwd", "softmax_attn_fwd", "sl_sample", "layer_fwd", "layer_bwd", "layer_append", "mfalcon_score", "abi_version", "last_error", "load_library",
           "HstuError", "LIB_PATH", "profile_enable", "profile_collect", "HSTU_BF16", "HSTU_F32", "HSTU_ACT_SILU", "HSTU_ACT_RELU"]
