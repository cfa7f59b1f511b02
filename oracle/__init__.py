"""fp64 CPU oracle for the gated delta rule.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the library.
"""
from .gdn_oracle import (  # noqa: F401
    decode_attention,
    dequantize_q4,
    gated_delta_chunk_form,
    gated_delta_decode_fused,
    gated_delta_decode_step,
    gated_delta_recurrence,
    grouped_gemm_q4,
    qk_head_of,
    round_bf16,
    sigmoid,
    softplus,
)
