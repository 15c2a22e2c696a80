"""CPU oracle (test infrastructure only; see siglip_oracle's header)."""
from .siglip_oracle import (  # noqa: F401
    LN_EPS, FP8_SCALE_EXP, E4M3_MAX, linear, layer_norm, gelu_tanh, softmax,
    attention, split_heads, merge_heads, e4m3_round, fp8_operand, weight_gemm, patch_embed,
    encoder_layer, map_head, encode,
)
