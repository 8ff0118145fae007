"""CPU fp64 oracle for causal scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the library.  See attention.py.
"""
from .attention import (  # noqa: F401
    attention_backward,
    attention_forward,
    attention_head,
    decode,
    decode_head,
    e4m3_decode,
    fp8qk_forward,
    gqa_backward,
    gqa_forward,
    head_backward,
    head_forward,
)
