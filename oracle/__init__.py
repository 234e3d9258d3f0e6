"""CPU oracle (test infrastructure only; see ``oracle.moe``)."""
from .moe import (  # noqa: F401
    fp16_bits_to_f64, bf16_bits_to_f64, dequant_q2k, dequant_cb2, dequant_matrix,
    router_logits, top_k, group_by_expert, silu, swiglu_ffn, Layer, moe_layer, moe_stack, rel_l2,
    rms_inv, RMS_EPS,
)
