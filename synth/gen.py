"""Seeded generators for the synthetic MoE workloads.

Every tensor of every layer comes from its own counter-keyed stream
``numpy.random.Generator(PCG64(SeedSequence([workload, layer, tensor, index])))``
so any expert of any layer can be regenerated alone, in any order, and the
bytes are identical on every machine with the same numpy.

What the streams hold (the recipe is the library's reading of the pages'
workload; the pages themselves print no weights):

* routed expert matrices: raw block bytes of the two 2-bit formats the
  QuarkStar and DwarfStar pages name for routed experts (QuarkStar README,
  "Model Weights": gate/up at a codebook 2-bit type, down at a Q2_K-type),
  with every quantised field uniform over its range and every fp16 scale
  drawn as fp16(U[0,1) * 2^-10), rounded to nearest even;
* the codebook: 256 rows x 8 entries, each uniform over {1, 3, 5, 7};
* router weights fp32 ~ N(0, 0.02^2); an optional Zipf(s) expert-popularity
  bias b[e] = -s * ln(1 + rank(e)) with rank a seeded permutation;
* the routed experts of a stack's tail layers (the pages' models with the
  last layers' experts at 4 bits) as Q4_K-style blocks, fields uniform and
  d, dmin = fp16(U[0,1) * 2^-14);
* the shared expert in bf16 ~ N(0, 0.02^2), rounded to nearest even;
* token activations fp32 ~ N(0, 1).

The module does no part of the MoE step's arithmetic.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np

# Block geometry of the two routed-expert formats (bytes per 256 weights).
Q2K_BLOCK_BYTES = 84
CB2_BLOCK_BYTES = 70
Q4K_BLOCK_BYTES = 144
BLOCK_WEIGHTS = 256
# 8-bit shared-expert blocks: 32 weights, fp16 scale + 32 int8 codes
Q8_BLOCK_BYTES = 34
Q8_BLOCK_WEIGHTS = 32

# Tensor ids used in the seed key.
T_ROUTER, T_BIAS, T_GATE, T_UP, T_DOWN, T_SGATE, T_SUP, T_SDOWN, T_X, T_CODEBOOK = range(10)


@dataclass(frozen=True)
class Workload:
    """Shapes, formats and router bias of one synthetic MoE workload."""

    name: str
    seed_id: int
    hidden: int            # H
    n_experts: int         # E
    top_k: int             # k
    expert_ffn: int        # F
    shared_ffn: int        # Fs (0 = no shared expert)
    gate_up_format: str    # "cb2" or "q2k"
    down_format: str       # "cb2" or "q2k"
    n_layers: int
    tokens: Tuple[int, ...] = (1,)
    zipf_s: Optional[float] = None
    note: str = ""
    shared_format: str = "bf16"   # "bf16" or "q8" (8-bit blocks of 32)
    tail_layers: int = 0          # the last tail_layers layers hold their experts as "q4k"

    def block_bytes(self, fmt: str) -> int:
        return block_bytes(fmt)

    def layer_formats(self, layer: int) -> Tuple[str, str]:
        """(gate/up format, down format) of a layer's routed experts."""
        if layer >= self.n_layers - self.tail_layers:
            return "q4k", "q4k"
        return self.gate_up_format, self.down_format

    def expert_bytes(self, layer: int = 0) -> Tuple[int, int, int]:
        """Bytes of one expert's gate, up and down matrices in the raw format
        (of layer `layer`)."""
        H, F = self.hidden, self.expert_ffn
        gf, df = self.layer_formats(layer)
        g = F * (H // BLOCK_WEIGHTS) * block_bytes(gf)
        d = H * (F // BLOCK_WEIGHTS) * block_bytes(df)
        return g, g, d

    def router_bytes(self) -> int:
        return self.n_experts * self.hidden * 4

    def shared_bytes(self) -> int:
        n = 3 * self.shared_ffn * self.hidden
        if self.shared_format == "q8":
            return n // Q8_BLOCK_WEIGHTS * Q8_BLOCK_BYTES
        return n * 2

    def stored_bytes(self) -> int:
        total = 0
        for l in range(self.n_layers):
            g, u, d = self.expert_bytes(l)
            total += self.n_experts * (g + u + d) + self.router_bytes() + self.shared_bytes()
        return total

    def step_bytes(self, distinct_experts_per_layer, n_tokens: int) -> int:
        """Algorithmic bytes one decode step must read and write: per layer the
        router, the shared expert and each distinct selected expert once, plus
        the activations in and out."""
        total = 0
        for l, u_l in enumerate(distinct_experts_per_layer):
            g, u, d = self.expert_bytes(l)
            total += self.router_bytes() + self.shared_bytes() + int(u_l) * (g + u + d)
        return total + 2 * n_tokens * self.hidden * 4


WORKLOADS = {
    # tiny single layer, every matrix Q2_K-style, no shared expert
    "tiny_q2k": Workload("tiny_q2k", 0, 512, 16, 2, 256, 0, "q2k", "q2k", 1, (1, 4, 16, 64),
                         note="tiny single layer, all Q2_K-style"),
    # Qwen3.6-35B-A3B-class single layer with a bf16 shared expert
    "a3b_layer": Workload("a3b_layer", 1, 2048, 256, 8, 512, 512, "cb2", "q2k", 1, (1,),
                          note="Qwen3.6-35B-A3B-class single layer"),
    # 40 routed-only layers of the A3B shapes, near-uniform picks
    "a3b_routed40": Workload("a3b_routed40", 2, 2048, 256, 8, 512, 0, "cb2", "q2k", 40, (1,),
                             note="40-layer routed-expert stack, A3B shapes"),
    # the same stack with every matrix Q2_K-style (secondary reading)
    "a3b_routed40_q2k": Workload("a3b_routed40_q2k", 5, 2048, 256, 8, 512, 0, "q2k", "q2k", 40, (1,),
                                 note="40-layer routed stack, all Q2_K-style"),
    # 40 layers of the single-layer shapes incl. shared expert, Zipf(1.1) router bias
    "a3b_stack40_zipf": Workload("a3b_stack40_zipf", 3, 2048, 256, 8, 512, 512, "cb2", "q2k", 40,
                                 (1, 4, 16, 64), zipf_s=1.1,
                                 note="40-layer A3B stack with shared expert, Zipf(1.1) popularity"),
    # the same with the shared expert in 8-bit blocks (the pages run every
    # non-routed tensor at Q8)
    "a3b_stack40_zipf_q8": Workload("a3b_stack40_zipf_q8", 6, 2048, 256, 8, 512, 512, "cb2", "q2k", 40,
                                    (1, 4), zipf_s=1.1, shared_format="q8",
                                    note="40-layer A3B stack, 8-bit shared expert, Zipf(1.1) popularity"),
    # the A3B stack with the last 6 layers' experts at a Q4_K type (the
    # pages' Layers34-39Q4KExperts model)
    "a3b_stack40_q4tail": Workload("a3b_stack40_q4tail", 7, 2048, 256, 8, 512, 512, "cb2", "q2k", 40,
                                   (1, 4, 16), zipf_s=1.1, tail_layers=6,
                                   note="40-layer A3B stack, layers 34-39 with Q4_K-style experts"),
    # DeepSeek-V4-Flash-class large layer, 8 stacked
    "flash_stack8_zipf": Workload("flash_stack8_zipf", 4, 4096, 256, 6, 2048, 2048, "cb2", "q2k", 8,
                                  (1, 8, 32), zipf_s=1.1,
                                  note="8-layer DeepSeek-V4-Flash-class stack, Zipf(1.1) popularity"),
}


def block_bytes(fmt: str) -> int:
    if fmt == "q2k":
        return Q2K_BLOCK_BYTES
    if fmt == "cb2":
        return CB2_BLOCK_BYTES
    if fmt == "q4k":
        return Q4K_BLOCK_BYTES
    raise ValueError(f"unknown block format {fmt!r}")


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def _fp16_scales(rng: np.random.Generator, n: int) -> np.ndarray:
    """n fp16 bit patterns of fp16(U[0,1) * 2^-10), round to nearest even."""
    u = rng.random(n, dtype=np.float32) * np.float32(2.0 ** -10)
    return u.astype(np.float16).view(np.uint16)


def fp32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest even) and return the 16-bit patterns."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def codebook(seed: int = 0) -> np.ndarray:
    """The 256 x 8 codebook of the codebook 2-bit format: int8 entries, each
    uniform over {1, 3, 5, 7}, row-major, from stream (seed, codebook)."""
    rng = _rng(seed, T_CODEBOOK)
    return (2 * rng.integers(0, 4, size=(256, 8)) + 1).astype(np.int8)


def _raw(rng, nblocks, bb, out):
    src = np.frombuffer(rng.bytes(nblocks * bb), dtype=np.uint8).reshape(nblocks, bb)
    if out is None:
        return src.copy()
    out = out.reshape(nblocks, bb)
    out[...] = src
    return out


def q2k_blocks(rng: np.random.Generator, nblocks: int, out=None) -> np.ndarray:
    """nblocks raw Q2_K-style blocks [nblocks][84]: bytes 0..79 (scales and
    2-bit codes) uniform, d and dmin (bytes 80..83) fp16(U[0,1)*2^-10)."""
    raw = _raw(rng, nblocks, Q2K_BLOCK_BYTES, out)
    dd = _fp16_scales(rng, 2 * nblocks).reshape(nblocks, 2)
    raw[:, 80:84] = dd.view(np.uint8).reshape(nblocks, 4)
    return raw


def cb2_blocks(rng: np.random.Generator, nblocks: int, out=None) -> np.ndarray:
    """nblocks raw codebook 2-bit blocks [nblocks][70]: d (bytes 0..1)
    fp16(U[0,1)*2^-10); scales, codebook indices and sign masks uniform."""
    raw = _raw(rng, nblocks, CB2_BLOCK_BYTES, out)
    d = _fp16_scales(rng, nblocks)
    raw[:, 0:2] = d.view(np.uint8).reshape(nblocks, 2)
    return raw


def q4k_blocks(rng: np.random.Generator, nblocks: int, out=None) -> np.ndarray:
    """nblocks raw Q4_K-style blocks [nblocks][144]: d (bytes 0..1) and dmin
    (2..3) fp16(U[0,1)*2^-14), every other byte uniform."""
    raw = out if out is not None else np.empty((nblocks, Q4K_BLOCK_BYTES), dtype=np.uint8)
    raw = raw.reshape(nblocks, Q4K_BLOCK_BYTES)
    raw[:] = np.frombuffer(rng.bytes(nblocks * Q4K_BLOCK_BYTES), dtype=np.uint8).reshape(nblocks, Q4K_BLOCK_BYTES)
    u = rng.random((nblocks, 2), dtype=np.float32) * np.float32(2.0 ** -14)
    raw[:, 0:4] = u.astype(np.float16).view(np.uint16).view(np.uint8).reshape(nblocks, 4)
    return raw


def q8_blocks(rng: np.random.Generator, nblocks: int) -> np.ndarray:
    """nblocks 8-bit blocks [nblocks][34]: d (bytes 0..1) fp16(U[0,1)*2^-11),
    then 32 int8 codes uniform over [-128, 127]."""
    raw = np.frombuffer(rng.bytes(nblocks * Q8_BLOCK_BYTES), dtype=np.uint8).reshape(nblocks, Q8_BLOCK_BYTES).copy()
    u = rng.random(nblocks, dtype=np.float32) * np.float32(2.0 ** -11)
    raw[:, 0:2] = u.astype(np.float16).view(np.uint16).view(np.uint8).reshape(nblocks, 2)
    return raw


def expert_tensor(wl: Workload, layer: int, tensor: int, expert: int, out=None) -> np.ndarray:
    """Raw bytes of one expert matrix, shape [rows][cols/256][block bytes]:
    gate/up are [F][H/256] blocks, down is [H][F/256] blocks."""
    H, F = wl.hidden, wl.expert_ffn
    gf, df = wl.layer_formats(layer)
    if tensor in (T_GATE, T_UP):
        rows, kb, fmt = F, H // BLOCK_WEIGHTS, gf
    elif tensor == T_DOWN:
        rows, kb, fmt = H, F // BLOCK_WEIGHTS, df
    else:
        raise ValueError("not an expert tensor")
    rng = _rng(wl.seed_id, layer, tensor, expert)
    gen = {"q2k": q2k_blocks, "cb2": cb2_blocks, "q4k": q4k_blocks}[fmt]
    return gen(rng, rows * kb, out).reshape(rows, kb, block_bytes(fmt))


@dataclass
class LayerWeights:
    """One layer's tensors in the raw (upload) layout."""

    router: np.ndarray                 # fp32 [E][H]
    router_bias: Optional[np.ndarray]  # fp32 [E] or None
    gate: np.ndarray                   # uint8 [E][F][H/256][bb]
    up: np.ndarray                     # uint8 [E][F][H/256][bb]
    down: np.ndarray                   # uint8 [E][H][F/256][bb]
    shared_gate: Optional[np.ndarray] = None   # bf16 bits [Fs][H], or 8-bit blocks [Fs][H/32][34]
    shared_up: Optional[np.ndarray] = None     # the same layout as shared_gate
    shared_down: Optional[np.ndarray] = None   # bf16 bits [H][Fs], or 8-bit blocks [H][Fs/32][34]
    experts: Tuple[int, ...] = field(default_factory=tuple)
    gate_up_format: Optional[str] = None       # this layer's routed formats
    down_format: Optional[str] = None


def layer_weights(wl: Workload, layer: int, experts=None) -> LayerWeights:
    """Generate one layer.  ``experts`` restricts the routed matrices to a
    subset (in the given order); the router and shared expert are whole."""
    E, H, Fs = wl.n_experts, wl.hidden, wl.shared_ffn
    ex = tuple(range(E)) if experts is None else tuple(int(e) for e in experts)
    router = _rng(wl.seed_id, layer, T_ROUTER, 0).standard_normal((E, H), dtype=np.float32)
    router *= np.float32(0.02)
    bias = None
    if wl.zipf_s is not None:
        rank = _rng(wl.seed_id, layer, T_BIAS, 0).permutation(E)
        bias = (-wl.zipf_s * np.log1p(rank.astype(np.float64))).astype(np.float32)
    H, F = wl.hidden, wl.expert_ffn
    gf, df = wl.layer_formats(layer)
    bg, bd = block_bytes(gf), block_bytes(df)
    gate = np.empty((len(ex), F, H // BLOCK_WEIGHTS, bg), dtype=np.uint8)
    up = np.empty_like(gate)
    down = np.empty((len(ex), H, F // BLOCK_WEIGHTS, bd), dtype=np.uint8)
    for i, e in enumerate(ex):
        expert_tensor(wl, layer, T_GATE, e, gate[i])
        expert_tensor(wl, layer, T_UP, e, up[i])
        expert_tensor(wl, layer, T_DOWN, e, down[i])
    lw = LayerWeights(router, bias, gate, up, down, experts=ex, gate_up_format=gf, down_format=df)
    if Fs and wl.shared_format == "q8":
        def q8(tid, rows, cols):
            return q8_blocks(_rng(wl.seed_id, layer, tid, 0), rows * cols // Q8_BLOCK_WEIGHTS).reshape(
                rows, cols // Q8_BLOCK_WEIGHTS, Q8_BLOCK_BYTES)
        lw.shared_gate = q8(T_SGATE, Fs, H)
        lw.shared_up = q8(T_SUP, Fs, H)
        lw.shared_down = q8(T_SDOWN, H, Fs)
    elif Fs:
        def bf16(tid, shape):
            a = _rng(wl.seed_id, layer, tid, 0).standard_normal(shape, dtype=np.float32)
            return fp32_to_bf16_bits(a * np.float32(0.02))
        lw.shared_gate = bf16(T_SGATE, (Fs, H))
        lw.shared_up = bf16(T_SUP, (Fs, H))
        lw.shared_down = bf16(T_SDOWN, (H, Fs))
    return lw


def hotlist(wl: Workload, layers) -> np.ndarray:
    """(layer, expert) pairs of the given layers, most popular first: the
    rank of the Zipf popularity bias (every layer's rank 0, then every
    layer's rank 1, ...); expert order without one.  int32 [n][2]."""
    layers = list(layers)
    order = []
    for l in layers:
        if wl.zipf_s is not None:
            rank = _rng(wl.seed_id, l, T_BIAS, 0).permutation(wl.n_experts)
            order.append(np.argsort(rank, kind="stable"))
        else:
            order.append(np.arange(wl.n_experts))
    out = [(l, int(order[i][r])) for r in range(wl.n_experts) for i, l in enumerate(layers)]
    return np.array(out, dtype=np.int32).reshape(-1, 2)


def tokens(wl: Workload, n_tokens: int, batch: int = 0) -> np.ndarray:
    """Token activations fp32 [T][H] ~ N(0, 1) for input batch ``batch``."""
    return _rng(wl.seed_id, 0xFFFF, T_X, n_tokens, batch).standard_normal(
        (n_tokens, wl.hidden), dtype=np.float32)
