"""ctypes binding of include/qs_moe.h: the same entry points, argument
marshalling only.  Every step of the MoE path runs in libqsmoe.so; there is
no Python or CPU fallback, and importing this module without the built
library raises."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# QSMOE_LIB_VARIANT=stamps selects the profiling build (phase stamps
# compiled in, see build.py); otherwise the library itself
LIB_PATH = os.path.join(_HERE, "libqsmoe_stamps.so" if os.environ.get("QSMOE_LIB_VARIANT") == "stamps"
                        else "libqsmoe.so")

QS_MOE_ABI_VERSION = 5
QS_OK, QS_E_INVAL, QS_E_NOMEM, QS_E_HIP, QS_E_STATE, QS_E_UNSUPPORTED = 0, -1, -2, -3, -4, -5
QS_FMT_BF16, QS_FMT_Q2K, QS_FMT_CB2, QS_FMT_Q8, QS_FMT_Q4K = 0, 1, 2, 3, 4
QS_DECODE_RESIDUAL = 1
QS_DECODE_RMSNORM = 2
QS_DECODE_STEER = 4
QS_DECODE_EXCLUSIVE = 8

FORMATS = {"bf16": QS_FMT_BF16, "q2k": QS_FMT_Q2K, "cb2": QS_FMT_CB2, "q8": QS_FMT_Q8, "q4k": QS_FMT_Q4K}

# Every function include/qs_moe.h declares.
EXPORTS = (
    "qs_moe_create", "qs_moe_upload", "qs_moe_decode", "qs_moe_decode_static", "qs_moe_sync_status", "qs_moe_set_wait_limit",
    "qs_moe_set_steering", "qs_moe_cache_sync", "qs_moe_cache_preload", "qs_moe_cache_stats", "qs_moe_cache_slots",
    "qs_moe_route", "qs_moe_dequant", "qs_moe_memory_bytes", "qs_moe_destroy", "qs_moe_status_string",
)


class QsMoeConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "abi_version", "hidden", "n_experts", "top_k", "expert_ffn", "shared_ffn",
        "gate_up_format", "down_format", "n_layers", "max_tokens", "mfma_min_tokens", "device",
        "shared_format", "tail_layers", "expert_paging", "resident_layers", "cache_slots")]


class QsMoeLayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "router", "router_bias", "gate", "up", "down", "shared_gate", "shared_up", "shared_down")]


class QsError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} returned {status} ({text})")
        self.status = status


def _load() -> ctypes.CDLL:
    # torch ships its own libamdhip64 (same soname, different file name).  Load
    # it before libqsmoe.so so that the library binds to that one runtime;
    # loading libqsmoe.so first would bring in a second HIP runtime when torch
    # is imported later, and the two cannot share the device.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950) first")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, u32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint32
    sigs = {
        "qs_moe_create": [ctypes.POINTER(QsMoeConfig), vp, ctypes.POINTER(vp)],
        "qs_moe_upload": [vp, i32, ctypes.POINTER(QsMoeLayerWeights), vp],
        "qs_moe_decode": [vp, i32, i32, vp, vp, i32, u32, vp, vp, vp],
        "qs_moe_decode_static": [vp, i32, i32, vp, vp, i32, u32, vp, vp, vp],
        "qs_moe_sync_status": [vp, vp],
        "qs_moe_set_wait_limit": [vp, ctypes.c_int32],
        "qs_moe_set_steering": [vp, vp, ctypes.c_float, vp],
        "qs_moe_cache_sync": [vp, vp],
        "qs_moe_cache_preload": [vp, vp, i32, vp],
        "qs_moe_cache_stats": [vp, vp],
        "qs_moe_cache_slots": [vp, vp],
        "qs_moe_route": [vp, i32, vp, i32, u32, vp, vp, vp, vp, vp],
        "qs_moe_dequant": [vp, i32, i32, i32, vp, vp],
        "qs_moe_memory_bytes": [vp, ctypes.POINTER(ctypes.c_uint64)],
        "qs_moe_destroy": [vp],
        "qs_moe_status_string": [i32],
    }
    for name, args in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name == "qs_moe_status_string" else ctypes.c_int
    return lib


LIB = _load()


def status_string(status: int) -> str:
    return LIB.qs_moe_status_string(int(status)).decode()


def check(fn: str, status: int) -> int:
    if status != QS_OK:
        raise QsError(fn, status, status_string(status))
    return status


def _ptr(a) -> int:
    """Address of a torch tensor, numpy array or integer (0 for None)."""
    if a is None:
        return 0
    if isinstance(a, int):
        return a
    if hasattr(a, "data_ptr"):
        return a.data_ptr()
    if hasattr(a, "ctypes"):
        if not a.flags["C_CONTIGUOUS"]:
            raise ValueError("numpy arrays passed to the library must be C-contiguous")
        return a.ctypes.data
    raise TypeError(f"cannot take the address of {type(a)}")


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_config(hidden, n_experts, top_k, expert_ffn, shared_ffn, gate_up_format, down_format,
                n_layers, max_tokens, mfma_min_tokens=0, device=-1, shared_format="bf16",
                tail_layers=0, expert_paging=0, resident_layers=0, cache_slots=0) -> QsMoeConfig:
    fmt = lambda f: FORMATS[f] if isinstance(f, str) else int(f)  # noqa: E731
    return QsMoeConfig(QS_MOE_ABI_VERSION, hidden, n_experts, top_k, expert_ffn, shared_ffn,
                       fmt(gate_up_format), fmt(down_format), n_layers, max_tokens,
                       mfma_min_tokens, device, fmt(shared_format), tail_layers,
                       expert_paging, resident_layers, cache_slots)


def qs_moe_create(cfg: QsMoeConfig, codebook=None) -> int:
    h = ctypes.c_void_p()
    check("qs_moe_create", LIB.qs_moe_create(ctypes.byref(cfg), _ptr(codebook), ctypes.byref(h)))
    return h.value


def qs_moe_upload(h: int, layer: int, router, router_bias, gate, up, down,
                  shared_gate=None, shared_up=None, shared_down=None, stream=None) -> None:
    w = QsMoeLayerWeights(*(_ptr(a) for a in (router, router_bias, gate, up, down,
                                               shared_gate, shared_up, shared_down)))
    check("qs_moe_upload", LIB.qs_moe_upload(h, layer, ctypes.byref(w), _stream(stream)))


def qs_moe_decode(h: int, layer0: int, n_layers: int, x, y, n_tokens: int, flags: int = 0,
                  ids_out=None, w_out=None, stream=None) -> None:
    check("qs_moe_decode", LIB.qs_moe_decode(h, layer0, n_layers, _ptr(x), _ptr(y), n_tokens,
                                             flags, _ptr(ids_out), _ptr(w_out), _stream(stream)))


def qs_moe_decode_static(h: int, layer0: int, n_layers: int, x, y, n_tokens: int, flags: int = 0,
                         ids_out=None, w_out=None, stream=None) -> None:
    check("qs_moe_decode_static", LIB.qs_moe_decode_static(h, layer0, n_layers, _ptr(x), _ptr(y), n_tokens,
                                                           flags, _ptr(ids_out), _ptr(w_out), _stream(stream)))


def qs_moe_sync_status(h: int, stream=None) -> None:
    check("qs_moe_sync_status", LIB.qs_moe_sync_status(h, _stream(stream)))


def qs_moe_set_wait_limit(h: int, polls: int) -> None:
    check("qs_moe_set_wait_limit", LIB.qs_moe_set_wait_limit(h, polls))


def qs_moe_set_steering(h: int, dirs, scale: float, stream=None) -> None:
    check("qs_moe_set_steering", LIB.qs_moe_set_steering(h, _ptr(dirs), scale, _stream(stream)))


def qs_moe_cache_sync(h: int, stream=None) -> None:
    check("qs_moe_cache_sync", LIB.qs_moe_cache_sync(h, _stream(stream)))


def qs_moe_cache_preload(h: int, keys, stream=None) -> None:
    """keys: numpy int32 [n][2] of (layer, expert), hottest first."""
    check("qs_moe_cache_preload", LIB.qs_moe_cache_preload(h, _ptr(keys), len(keys), _stream(stream)))


def qs_moe_cache_stats(h: int, out) -> None:
    """out: numpy uint64 [8]."""
    check("qs_moe_cache_stats", LIB.qs_moe_cache_stats(h, _ptr(out)))


def qs_moe_cache_slots(h: int, out) -> None:
    """out: numpy int32 [cache_slots][2]."""
    check("qs_moe_cache_slots", LIB.qs_moe_cache_slots(h, _ptr(out)))


def qs_moe_route(h: int, layer: int, x, n_tokens: int, flags: int = 0, logits_out=None,
                 ids_out=None, w_out=None, group_out=None, stream=None) -> None:
    check("qs_moe_route", LIB.qs_moe_route(h, layer, _ptr(x), n_tokens, flags, _ptr(logits_out),
                                           _ptr(ids_out), _ptr(w_out), _ptr(group_out),
                                           _stream(stream)))


def qs_moe_dequant(h: int, layer: int, expert: int, which: int, out, stream=None) -> None:
    check("qs_moe_dequant", LIB.qs_moe_dequant(h, layer, expert, which, _ptr(out), _stream(stream)))


def qs_moe_memory_bytes(h: int) -> int:
    v = ctypes.c_uint64()
    check("qs_moe_memory_bytes", LIB.qs_moe_memory_bytes(h, ctypes.byref(v)))
    return v.value


def qs_moe_destroy(h: int) -> None:
    check("qs_moe_destroy", LIB.qs_moe_destroy(h))
