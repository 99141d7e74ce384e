"""CPU oracle of the Qwen3 attention block -- test infrastructure only.

Importable only from tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg.  The product path never imports it.
"""
from .qwen3_attn_oracle import (  # noqa: F401
    decode, decode_residual, gqa_attention, linear, merge_heads, prefill, prefill_chunk,
    prefill_residual, prefill_rows, project_norm_rope,
    rms_norm, rope, rope_inv_freq, softmax, split_heads,
)
