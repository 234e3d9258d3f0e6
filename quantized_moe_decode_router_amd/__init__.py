"""MI355X-native decode-time routed-expert MoE over 2-bit block weights.

The compute path is libqsmoe.so (hand-written HIP for gfx950) behind the C ABI
of include/qs_moe.h; this package is its ctypes binding plus a small handle
class that marshals torch tensors and numpy arrays.  PyTorch is used only
for device memory and streams.
"""
from ._lib import (  # noqa: F401
    LIB, LIB_PATH, EXPORTS, QsError, QsMoeConfig, QsMoeLayerWeights, status_string, make_config,
    qs_moe_create, qs_moe_upload, qs_moe_decode, qs_moe_decode_static, qs_moe_sync_status, qs_moe_set_wait_limit,
    qs_moe_set_steering, qs_moe_route, qs_moe_dequant,
    qs_moe_memory_bytes, qs_moe_destroy,
    QS_OK, QS_E_INVAL, QS_E_NOMEM, QS_E_HIP, QS_E_STATE, QS_E_UNSUPPORTED,
    QS_FMT_BF16, QS_FMT_Q2K, QS_FMT_CB2, QS_FMT_Q8, QS_FMT_Q4K, QS_DECODE_RESIDUAL, QS_DECODE_RMSNORM, QS_DECODE_STEER, QS_DECODE_EXCLUSIVE,
    QS_MOE_ABI_VERSION,
)
from .handle import MoE  # noqa: F401
