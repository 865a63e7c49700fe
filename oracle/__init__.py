"""fp64 CPU oracle for multi-head scaled dot-product attention.

Test infrastructure: only tests/, the smoke check and the bench's CPU-baseline
leg may import this package. The product path never does.
"""
from .attention_ref import (attention_backward_ref, attention_backward_sampled_ref, attention_ref,
                            attention_weights_ref, causal_mask, causal_mask_rows, decode_ref, encoder_layer_ref,
                            ffn_ref, gather_pages, key_padding_mask_row, layer_norm_ref, linear_ref, mha_ref,
                            softmax_rows)

__all__ = ["attention_backward_ref", "attention_backward_sampled_ref", "attention_ref", "attention_weights_ref",
           "causal_mask", "causal_mask_rows", "decode_ref", "encoder_layer_ref", "ffn_ref", "gather_pages",
           "key_padding_mask_row", "layer_norm_ref", "linear_ref", "mha_ref", "softmax_rows"]
