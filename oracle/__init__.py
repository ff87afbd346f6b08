"""CPU oracle (test infrastructure only).

Plain float64 numpy implementation of THD varlen attention forward and
backward.  Only the tests, ``__graft_entry__.smoke()`` and the benchmark's
CPU-baseline leg may import it; the GPU library never does.
"""
from .attention import (allowed_mask, attn_bwd, attn_bwd_seq, attn_fwd, attn_fwd_seq,
                        merge_partials, sequence_slots)
from .fp8 import attn_bwd_fp8, attn_fwd_fp8, decode_e4m3

__all__ = ["allowed_mask", "attn_bwd", "attn_bwd_seq", "attn_fwd", "attn_fwd_seq",
           "merge_partials", "sequence_slots", "attn_fwd_fp8", "attn_bwd_fp8", "decode_e4m3"]
