"""CPU oracle for exact attention (test infrastructure only).

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this package; the HIP product path never does.
"""
from .attention import (attn_ref_bwd, attn_ref_bwd_head, attn_ref_decode, attn_ref_fwd,
                        attn_ref_head, attn_ref_rows, dequant_fp8, e4m3_decode, kv_head, mask,
                        scores, softmax_three_pass)

__all__ = ["attn_ref_fwd", "attn_ref_bwd", "attn_ref_head", "attn_ref_bwd_head",
           "attn_ref_rows", "attn_ref_decode", "dequant_fp8", "e4m3_decode", "kv_head",
           "scores", "mask",
           "softmax_three_pass"]
