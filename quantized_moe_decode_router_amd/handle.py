"""A thin owner of one qs_moe handle: torch tensors in, torch tensors out.
Marshalling only; all compute is in libqsmoe.so."""
from __future__ import annotations

import numpy as np

from . import _lib as L


class MoE:
    """qs_moe handle for one model configuration on the current HIP device."""

    def __init__(self, hidden, n_experts, top_k, expert_ffn, shared_ffn, gate_up_format,
                 down_format, n_layers, max_tokens, codebook=None, mfma_min_tokens=0, device=-1,
                 shared_format="bf16", tail_layers=0, resident_layers=None, cache_slots=0):
        """resident_layers: None = every layer resident; else expert paging
        with that many leading resident layers and `cache_slots` HBM slots."""
        paging = resident_layers is not None
        self.cfg = L.make_config(hidden, n_experts, top_k, expert_ffn, shared_ffn, gate_up_format,
                                 down_format, n_layers, max_tokens, mfma_min_tokens, device,
                                 shared_format, tail_layers, int(paging),
                                 resident_layers if paging else 0, cache_slots if paging else 0)
        cb = None if codebook is None else np.ascontiguousarray(codebook, dtype=np.int8)
        self._cb = cb
        self.h = L.qs_moe_create(self.cfg, cb)

    @classmethod
    def for_workload(cls, wl, codebook, n_layers=None, max_tokens=64, **kw):
        """A handle for the first n_layers layers of a synthetic workload (its
        Q4_K-style tail layers among them, if any)."""
        n = n_layers or wl.n_layers
        tail = max(0, n - (wl.n_layers - getattr(wl, "tail_layers", 0)))
        return cls(wl.hidden, wl.n_experts, wl.top_k, wl.expert_ffn, wl.shared_ffn,
                   wl.gate_up_format, wl.down_format, n, max_tokens,
                   codebook=codebook, shared_format=getattr(wl, "shared_format", "bf16"),
                   tail_layers=tail, **kw)

    # -- lifetime ---------------------------------------------------------
    def close(self):
        if getattr(self, "h", None):
            L.qs_moe_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    # -- calls ------------------------------------------------------------
    def upload(self, layer, lw, stream=None):
        """Upload a synth.LayerWeights-like object (numpy, host memory)."""
        c = np.ascontiguousarray
        L.qs_moe_upload(self.h, layer, c(lw.router), None if lw.router_bias is None else c(lw.router_bias),
                        c(lw.gate), c(lw.up), c(lw.down),
                        None if lw.shared_gate is None else c(lw.shared_gate),
                        None if lw.shared_up is None else c(lw.shared_up),
                        None if lw.shared_down is None else c(lw.shared_down), stream)

    def decode(self, x, y=None, layer0=0, n_layers=1, residual=False, prenorm=False, ids_out=None,
               w_out=None, stream=None, steer=False, exclusive=False):
        """One qs_moe_decode call (one persistent kernel launch) on `stream`
        (torch's current stream by default); asynchronous.  exclusive: the
        caller runs nothing else on the device meanwhile (QS_DECODE_EXCLUSIVE)."""
        import torch
        T = x.shape[0]
        if y is None:
            y = torch.empty_like(x)
        flags = ((L.QS_DECODE_RESIDUAL if residual else 0) | (L.QS_DECODE_RMSNORM if prenorm else 0)
                 | (L.QS_DECODE_STEER if steer else 0) | (L.QS_DECODE_EXCLUSIVE if exclusive else 0))
        L.qs_moe_decode(self.h, layer0, n_layers, x, y, T, flags, ids_out, w_out, stream)
        return y

    def decode_static(self, x, y=None, layer0=0, n_layers=1, residual=False, prenorm=False, ids_out=None,
                      w_out=None, stream=None, steer=False, exclusive=False):
        """qs_moe_decode_static: decode with the library's static device scratch."""
        import torch
        T = x.shape[0]
        if y is None:
            y = torch.empty_like(x)
        flags = ((L.QS_DECODE_RESIDUAL if residual else 0) | (L.QS_DECODE_RMSNORM if prenorm else 0)
                 | (L.QS_DECODE_STEER if steer else 0) | (L.QS_DECODE_EXCLUSIVE if exclusive else 0))
        L.qs_moe_decode_static(self.h, layer0, n_layers, x, y, T, flags, ids_out, w_out, stream)
        return y

    def sync_status(self, stream=None):
        """Synchronise the stream; raise QsError (QS_E_HIP) if a decode call
        since the last check gave up a bounded wait."""
        L.qs_moe_sync_status(self.h, stream)

    def set_wait_limit(self, polls):
        L.qs_moe_set_wait_limit(self.h, polls)

    def set_steering(self, dirs, scale=1.0, stream=None):
        """qs_moe_set_steering: directions fp32 [n_layers][H] (numpy or torch,
        host or device), or None to clear them."""
        if dirs is not None and not hasattr(dirs, "data_ptr"):
            dirs = np.ascontiguousarray(dirs, dtype=np.float32)
        self._steer = dirs      # keeps a host array alive across the call
        L.qs_moe_set_steering(self.h, dirs, float(scale), stream)

    def route(self, x, layer=0, prenorm=False, stream=None):
        import torch
        T = x.shape[0]
        E, k = self.cfg.n_experts, self.cfg.top_k
        dev = x.device
        logits = torch.empty((T, E), dtype=torch.float64, device=dev)
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        w = torch.empty((T, k), dtype=torch.float32, device=dev)
        grp = torch.empty(3 * E + 2 + T * k, dtype=torch.int32, device=dev)
        L.qs_moe_route(self.h, layer, x, T, L.QS_DECODE_RMSNORM if prenorm else 0, logits, ids, w,
                       grp, stream)
        P = T * k
        return {
            "logits": logits, "ids": ids, "w": w,
            "counts": grp[:E], "offsets": grp[E:2 * E + 1], "pairs": grp[2 * E + 1:2 * E + 1 + P],
            "n_active": grp[2 * E + 1 + P], "active": grp[2 * E + 2 + P:],
        }

    def dequant(self, layer, expert, which, stream=None):
        """which: 0..2 routed gate/up/down of `expert`, 3..5 shared gate/up/down."""
        import torch
        H, F, Fs = self.cfg.hidden, self.cfg.expert_ffn, self.cfg.shared_ffn
        shape = {0: (F, H), 1: (F, H), 2: (H, F), 3: (Fs, H), 4: (Fs, H), 5: (H, Fs)}[which]
        out = torch.empty(shape, dtype=torch.float32, device="cuda")
        L.qs_moe_dequant(self.h, layer, expert, which, out, stream)
        return out

    # -- expert cache (expert paging) ---------------------------------------
    def cache_sync(self, stream=None):
        L.qs_moe_cache_sync(self.h, stream)

    def cache_preload(self, keys, stream=None):
        """keys: (layer, expert) pairs, hottest first."""
        k = np.ascontiguousarray(np.asarray(keys, dtype=np.int32).reshape(-1, 2))
        L.qs_moe_cache_preload(self.h, k, stream)

    CACHE_STATS = ("hits", "misses", "admissions", "evictions", "preloaded", "slots_used", "slots",
                   "host_bytes")

    def cache_stats(self):
        out = np.zeros(8, dtype=np.uint64)
        L.qs_moe_cache_stats(self.h, out)
        return {n: int(v) for n, v in zip(self.CACHE_STATS, out)}

    def cache_slots(self):
        """(layer, expert) per slot, (-1, -1) when free: numpy int32 [slots][2]."""
        out = np.zeros((max(self.cfg.cache_slots, 1), 2), dtype=np.int32)
        L.qs_moe_cache_slots(self.h, out)
        return out[:self.cfg.cache_slots]

    def memory_bytes(self):
        return L.qs_moe_memory_bytes(self.h)
