"""C-ABI checks that need no GPU: the library loads, exports every function
include/qs_moe.h declares, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

import quantized_moe_decode_router_amd as qm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qs_moe.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qs_moe_\w+)\s*\(", text)))


def test_header_and_binding_agree():
    assert header_functions() == sorted(qm.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(qm.LIB_PATH)
    for name in header_functions():
        assert hasattr(lib, name), name


def test_no_other_exported_qs_symbols():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", qm.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = sorted({l.split()[-1] for l in out.splitlines() if " T " in l and "qs_" in l})
    assert exported == header_functions()


def test_header_constants_match_binding():
    text = open(HEADER).read()
    defs = dict(re.findall(r"#define\s+(QS_\w+)\s+(\d+)u?\b", text))
    for name in ("QS_MOE_ABI_VERSION", "QS_DECODE_RESIDUAL", "QS_DECODE_RMSNORM", "QS_DECODE_STEER",
                 "QS_DECODE_EXCLUSIVE"):
        assert hasattr(qm, name), name
        assert int(defs[name]) == getattr(qm, name), name


def test_header_formats_match_binding():
    text = open(HEADER).read()
    enum = re.search(r"typedef enum \{([^}]*)\} qs_format;", text).group(1)
    vals = {n: int(v) for n, v in re.findall(r"(QS_FMT_\w+)\s*=\s*(\d+)", enum)}
    assert vals == {"QS_FMT_BF16": qm.QS_FMT_BF16, "QS_FMT_Q2K": qm.QS_FMT_Q2K,
                    "QS_FMT_CB2": qm.QS_FMT_CB2, "QS_FMT_Q8": qm.QS_FMT_Q8, "QS_FMT_Q4K": qm.QS_FMT_Q4K}
    # the config struct's fields, in the header's order
    body = re.search(r"typedef struct \{([^}]*)\} qs_moe_config;", text).group(1)
    names = re.findall(r"int32_t\s+(\w+);", body)
    assert names == [f for f, _ in qm.QsMoeConfig._fields_]


def test_status_strings():
    assert qm.status_string(qm.QS_OK) == "ok"
    for s in (qm.QS_E_INVAL, qm.QS_E_NOMEM, qm.QS_E_HIP, qm.QS_E_STATE, qm.QS_E_UNSUPPORTED):
        assert qm.status_string(s) not in ("ok", "unknown status")
    assert qm.status_string(12345) == "unknown status"


def _good():
    return dict(hidden=512, n_experts=16, top_k=2, expert_ffn=256, shared_ffn=0,
                gate_up_format="q2k", down_format="q2k", n_layers=1, max_tokens=4)


@pytest.mark.parametrize("field,value", [
    ("hidden", 0), ("hidden", 300), ("hidden", 32768), ("expert_ffn", 100), ("expert_ffn", 0),
    ("n_experts", 0), ("n_experts", 2048), ("top_k", 0), ("top_k", 17), ("top_k", 32),
    ("shared_ffn", -64), ("shared_ffn", 100), ("gate_up_format", 7), ("down_format", 0),
    ("n_layers", 0), ("max_tokens", 0), ("max_tokens", 257), ("mfma_min_tokens", -1),
    ("shared_format", 1), ("shared_format", 2), ("shared_format", 4), ("shared_format", -1),
    ("tail_layers", -1), ("tail_layers", 2),
    ("expert_paging", 2), ("expert_paging", -1), ("resident_layers", 1), ("cache_slots", 3),
])
def test_create_rejects_invalid_config_without_gpu(field, value):
    kw = _good()
    kw[field] = value
    cfg = qm.make_config(**kw)
    h = ctypes.c_void_p(123)
    rc = qm.LIB.qs_moe_create(ctypes.byref(cfg), None, ctypes.byref(h))
    assert rc == qm.QS_E_INVAL
    assert h.value is None


@pytest.mark.parametrize("resident,slots", [(-1, 0), (3, 0), (0, -1), (0, 33), (1, 17), (2, 1)])
def test_create_rejects_invalid_paging_without_gpu(resident, slots):
    """With paging on: 0 <= resident_layers <= n_layers, and at most one
    slot per paged expert (2 layers of 16 experts here)."""
    kw = _good()
    kw.update(n_layers=2, expert_paging=1, resident_layers=resident, cache_slots=slots)
    cfg = qm.make_config(**kw)
    h = ctypes.c_void_p(123)
    assert qm.LIB.qs_moe_create(ctypes.byref(cfg), None, ctypes.byref(h)) == qm.QS_E_INVAL
    assert h.value is None


def test_create_rejects_bad_abi_version_and_pair_budget():
    cfg = qm.make_config(**_good())
    cfg.abi_version = 99
    h = ctypes.c_void_p()
    assert qm.LIB.qs_moe_create(ctypes.byref(cfg), None, ctypes.byref(h)) == qm.QS_E_INVAL
    kw = _good()
    kw.update(n_experts=64, top_k=8, max_tokens=256)       # 2048 pairs > 1024
    cfg = qm.make_config(**kw)
    assert qm.LIB.qs_moe_create(ctypes.byref(cfg), None, ctypes.byref(h)) == qm.QS_E_INVAL


def test_create_requires_codebook_for_codebook_format():
    kw = _good()
    kw["gate_up_format"] = "cb2"
    cfg = qm.make_config(**kw)
    h = ctypes.c_void_p()
    assert qm.LIB.qs_moe_create(ctypes.byref(cfg), None, ctypes.byref(h)) == qm.QS_E_INVAL


def test_codebook_down_format_is_unsupported():
    kw = _good()
    kw["down_format"] = "cb2"
    cfg = qm.make_config(**kw)
    h = ctypes.c_void_p()
    cb = (ctypes.c_int8 * 2048)()
    assert qm.LIB.qs_moe_create(ctypes.byref(cfg), cb, ctypes.byref(h)) == qm.QS_E_UNSUPPORTED


def test_null_arguments():
    assert qm.LIB.qs_moe_create(None, None, None) == qm.QS_E_INVAL
    h = ctypes.c_void_p()
    assert qm.LIB.qs_moe_create(None, None, ctypes.byref(h)) == qm.QS_E_INVAL
    assert qm.LIB.qs_moe_destroy(None) == qm.QS_OK
    assert qm.LIB.qs_moe_decode(None, 0, 1, None, None, 1, 0, None, None, None) == qm.QS_E_INVAL
    assert qm.LIB.qs_moe_upload(None, 0, None, None) == qm.QS_E_INVAL
    assert qm.LIB.qs_moe_route(None, 0, None, 1, 0, None, None, None, None, None) == qm.QS_E_INVAL
    assert qm.LIB.qs_moe_dequant(None, 0, 0, 0, None, None) == qm.QS_E_INVAL
    assert qm.LIB.qs_moe_memory_bytes(None, None) == qm.QS_E_INVAL
    assert qm.LIB.qs_moe_sync_status(None, None) == qm.QS_E_INVAL
    assert qm.LIB.qs_moe_set_wait_limit(None, 0) == qm.QS_E_INVAL
    assert qm.LIB.qs_moe_cache_sync(None, None) == qm.QS_E_INVAL
    assert qm.LIB.qs_moe_cache_preload(None, None, 0, None) == qm.QS_E_INVAL
    assert qm.LIB.qs_moe_cache_stats(None, None) == qm.QS_E_INVAL
    assert qm.LIB.qs_moe_cache_slots(None, None) == qm.QS_E_INVAL
