"""fp64 CPU oracle for the attention path.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product library or its binding.
"""

from .attention import (apply_rope, apply_rope_transpose, attention, attention_backward, attention_backward_sampled,
                        attention_fp8, attention_rows, causal_mask, decode_paged, fp8_e4m3_decode, gather_paged,
                        kv_head_of, max_abs, prefill_paged, rel_rms, rope_inv_freq, sdpa, window_mask)

__all__ = ["apply_rope", "apply_rope_transpose", "attention", "attention_backward", "attention_backward_sampled",
           "attention_fp8", "attention_rows", "causal_mask", "decode_paged", "fp8_e4m3_decode", "gather_paged",
           "kv_head_of", "max_abs", "prefill_paged", "rel_rms", "rope_inv_freq", "sdpa", "window_mask"]
