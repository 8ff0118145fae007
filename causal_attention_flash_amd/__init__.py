"""Fused causal scaled-dot-product attention for AMD Instinct MI355X (gfx950).

Python binding of the C ABI in include/attn.h (libcausal_attn.so, hand-written
HIP kernels).  The binding marshals torch tensors to pointers and the current
stream; all computation runs in the library's kernels.

    o, lse = attn_fwd(q, k, v, scale=None, causal=True)
    dq, dk, dv = attn_bwd(q, k, v, o, do, lse, scale=None, causal=True)
    dq, dk, dv = attn_bwd_atomic(q, k, v, o, do, lse)  # dQ by fp32 atomics (D = 64)
    o, lse = attn_fwd_gqa(q, k, v)          # K, V with fewer (grouped) heads
    dq, dk, dv = attn_bwd_gqa(q, k, v, o, do, lse)
    o, lse = attn_decode(q, k_cache, v_cache, kv_lens=None)  # one query row per head
    o, lse = attn_fwd_fp8qk(q8, k8, v, q_descale, k_descale)  # fp8 (E4M3) Q and K
"""
from ._binding import (  # noqa: F401
    ATTN_BF16,
    ATTN_F16,
    ATTN_F32,
    LIB_PATH,
    SIGNATURES,
    STATUS_NAMES,
    AttnError,
    attn_bwd,
    attn_bwd_atomic,
    attn_bwd_dkdv,
    attn_bwd_dq,
    attn_bwd_dq_delta,
    attn_bwd_gqa,
    attn_bwd_preprocess,
    attn_decode,
    attn_fwd,
    attn_fwd_fp8qk,
    attn_fwd_gqa,
    load_library,
    status_string,
)
