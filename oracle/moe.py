"""CPU oracle of the decode-time routed-expert MoE step over 2-bit block weights.

TEST INFRASTRUCTURE.  This module is the plain, slow definition the HIP
library is checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import it; the library and its
Python binding never do, and it shares no code with them.

What it computes and where that comes from
------------------------------------------
* The recipe: only the routed experts are quantised to 2 bits (gate/up at a
  codebook type, down at a Q2_K type); the shared expert, projections and the
  router stay at high precision (QuarkStar README, "Model Weights";
  DwarfStar page, "Model Weights").
* Dequantisation fused into the matrix-vector products of single-stream
  decode (Quasar README, "Design decisions" and "Performance model").
* Optional directional steering of each layer's FFN output,
  m - scale * d * (d . m), before the residual add (QuarkStar README,
  "Steering").
* The pages name the block types but print no layout, no router equations
  and no layer shapes.  The block layouts below, softmax-then-top-k with
  renormalisation, ties to the lower expert index, an ungated shared expert
  and the residual chaining of stacked layers are this library's readings;
  each is stated where it is used.

Precision: every floating-point step is fp64 over exact fp32/fp16/bf16
inputs.  The dequantised weight is the exact value of its formula rounded
once to fp32 (the value the library stores).  Router logits are fp64 sums of
exact fp32 x fp32 products, so top-k decisions are taken in fp64 on both
sides.  The layer output is rounded to fp32 once, at the end.

Every function here is pinned by ``tests/test_oracle_*.py`` against closed
forms, library routines on special cases, invariants or brute force.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------- scalars ---


def fp16_bits_to_f64(bits) -> np.ndarray:
    """IEEE 754 binary16 bit patterns -> exact float64 values.

    From the definition: sign s, exponent e (5 bits, bias 15), fraction m
    (10 bits).  e = 0: (-1)^s * m * 2^-24 (zero and subnormals);
    0 < e < 31: (-1)^s * (1024 + m) * 2^(e-25); e = 31: inf (m = 0) or NaN.
    """
    b = np.asarray(bits).astype(np.int64)
    s = (b >> 15) & 1
    e = (b >> 10) & 0x1F
    m = b & 0x3FF
    mag = np.where(e == 0, m * 2.0 ** -24, (1024 + m) * np.exp2(e.astype(np.float64) - 25))
    mag = np.where(e == 31, np.where(m == 0, np.inf, np.nan), mag)
    return np.where(s == 1, -mag, mag)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns -> float64: the pattern is the top half of an
    IEEE binary32, so the value is that of ``bits << 16`` read as fp32."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):        # NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)


# --------------------------------------------------------------- formats ---
# Q2_K-style block, 84 bytes per 256 weights (the Q2_K type the QuarkStar and
# DwarfStar pages use for routed down projections; layout is this library's):
#   bytes  0..15  scales[16]: sub-block i (weights 16i..16i+15) has
#                 sc = low nibble, m = high nibble
#   bytes 16..79  qs[64]: weight j has q = (qs[j // 4] >> (2 * (j % 4))) & 3
#   bytes 80..81  d    (fp16, little endian)
#   bytes 82..83  dmin (fp16, little endian)
#   w_j = d * sc * q_j - dmin * m
#
# Codebook 2-bit block, 70 bytes per 256 weights (the IQ2_XXS-type role for
# routed gate/up; layout is this library's):
#   bytes  0..1   d (fp16)
#   bytes  2..5   scales: sub-block i (weights 32i..32i+31) has
#                 s = (byte[2 + i // 2] >> (4 * (i % 2))) & 15
#   bytes  6..37  idx[32]: group g (weights 8g..8g+7) uses codebook row idx[g]
#   bytes 38..69  sign[32]: bit b of sign[g] set => weight 8g+b is negative
#   w_j = d * s * C[idx[j // 8]][j % 8], negated if its sign bit is set


def dequant_q2k(blocks: np.ndarray) -> np.ndarray:
    """Raw Q2_K-style blocks [..., 84] uint8 -> fp32 weights [..., 256]."""
    blk = np.asarray(blocks, dtype=np.uint8)
    lead = blk.shape[:-1]
    blk = blk.reshape(-1, 84)
    j = np.arange(256)
    sub = blk[:, 0:16][:, j // 16].astype(np.int64)           # scale byte of each weight
    sc = sub & 0xF
    m = sub >> 4
    q = (blk[:, 16:80][:, j // 4].astype(np.int64) >> (2 * (j % 4))) & 3
    d = fp16_bits_to_f64(blk[:, 80].astype(np.uint16) | (blk[:, 81].astype(np.uint16) << 8))[:, None]
    dmin = fp16_bits_to_f64(blk[:, 82].astype(np.uint16) | (blk[:, 83].astype(np.uint16) << 8))[:, None]
    # exact in fp64 (products <= 17 significant bits, difference of two
    # multiples of 2^-24 below 2^21), then one rounding to fp32
    w = d * sc * q - dmin * m
    return w.astype(np.float32).reshape(*lead, 256)


def dequant_cb2(blocks: np.ndarray, codebook: np.ndarray) -> np.ndarray:
    """Raw codebook 2-bit blocks [..., 70] uint8 -> fp32 weights [..., 256]."""
    blk = np.asarray(blocks, dtype=np.uint8)
    cb = np.asarray(codebook, dtype=np.int64).reshape(256, 8)
    lead = blk.shape[:-1]
    blk = blk.reshape(-1, 70)
    j = np.arange(256)
    d = fp16_bits_to_f64(blk[:, 0].astype(np.uint16) | (blk[:, 1].astype(np.uint16) << 8))[:, None]
    i = j // 32
    s = (blk[:, 2:6][:, i // 2].astype(np.int64) >> (4 * (i % 2))) & 0xF
    g = j // 8
    c = cb[blk[:, 6:38][:, g].astype(np.int64), j % 8]
    neg = (blk[:, 38:70][:, g].astype(np.int64) >> (j % 8)) & 1
    w = d * s * c                                            # exact: <= 18 significant bits
    w = np.where(neg == 1, -w, w)
    return w.astype(np.float32).reshape(*lead, 256)


# Q4_K-style block, 144 bytes per 256 weights (the 4-bit type the pages keep
# the routed experts of the last layers at -- QuarkStar README, "Model
# Weights": the Layers34-39Q4KExperts model; DwarfStar page, "Model
# Weights": q2 with the last 6 layers at q4):
#   bytes 0..1    d (fp16)          bytes 2..3   dmin (fp16)
#   bytes 4..15   scales[12]: eight 6-bit (sc, m) pairs, one per 32-weight
#                 sub-block j:  j < 4:  sc = scales[j] & 63,
#                                       m  = scales[j + 4] & 63
#                               j >= 4: sc = (scales[j + 4] & 15) | (scales[j - 4] >> 6) << 4,
#                                       m  = (scales[j + 4] >> 4) | (scales[j] >> 6) << 4
#   bytes 16..143 qs[128]: weights 64c + r of chunk c = 0..3 take the low
#                 nibble of qs[32c + r] for r < 32, the high nibble of
#                 qs[32c + r - 32] for r >= 32
#   w_j = d * sc * q_j - dmin * m   (sc, m of sub-block j // 32)


def q4k_scales(scales: np.ndarray):
    """12 packed scale bytes [..., 12] -> (sc [..., 8], m [..., 8]) as int64."""
    b = np.asarray(scales, dtype=np.int64)
    sc = np.empty(b.shape[:-1] + (8,), dtype=np.int64)
    m = np.empty_like(sc)
    for j in range(8):
        if j < 4:
            sc[..., j] = b[..., j] & 63
            m[..., j] = b[..., j + 4] & 63
        else:
            sc[..., j] = (b[..., j + 4] & 15) | ((b[..., j - 4] >> 6) << 4)
            m[..., j] = (b[..., j + 4] >> 4) | ((b[..., j] >> 6) << 4)
    return sc, m


def dequant_q4k(blocks: np.ndarray) -> np.ndarray:
    """Raw Q4_K-style blocks [..., 144] uint8 -> fp32 weights [..., 256]."""
    blk = np.asarray(blocks, dtype=np.uint8)
    lead = blk.shape[:-1]
    blk = blk.reshape(-1, 144)
    d = fp16_bits_to_f64(blk[:, 0].astype(np.uint16) | (blk[:, 1].astype(np.uint16) << 8))[:, None]
    dmin = fp16_bits_to_f64(blk[:, 2].astype(np.uint16) | (blk[:, 3].astype(np.uint16) << 8))[:, None]
    sc, m = q4k_scales(blk[:, 4:16])
    j = np.arange(256)
    c, r = j // 64, j % 64
    byte = blk[:, 16:144][:, 32 * c + (r % 32)].astype(np.int64)
    q = np.where(r < 32, byte & 15, byte >> 4)
    sub = j // 32
    # exact in fp64 (products of at most 21 significant bits), then one
    # rounding to fp32
    w = d * sc[:, sub] * q - dmin * m[:, sub]
    return w.astype(np.float32).reshape(*lead, 256)


# 8-bit block, 34 bytes per 32 weights (the Q8_0 type the pages use for the
# tensors they keep at 8 bits -- QuarkStar README, "Model Weights" (Q8 rest);
# DwarfStar page, "Distributed Inference" (Q8 shared experts)):
#   bytes 0..1   d (fp16)
#   bytes 2..33  qs[32]: int8 codes
#   w_j = d * qs[j]


def dequant_q8(blocks: np.ndarray) -> np.ndarray:
    """Raw 8-bit blocks [..., 34] uint8 -> fp32 weights [..., 32] (exact:
    an 11-bit significand times an 8-bit integer fits fp32)."""
    blk = np.asarray(blocks, dtype=np.uint8)
    lead = blk.shape[:-1]
    blk = blk.reshape(-1, 34)
    d = fp16_bits_to_f64(blk[:, 0].astype(np.uint16) | (blk[:, 1].astype(np.uint16) << 8))[:, None]
    q = blk[:, 2:34].view(np.int8).astype(np.float64)
    return (d * q).astype(np.float32).reshape(*lead, 32)


def dequant_matrix(raw: np.ndarray, fmt: str, codebook=None) -> np.ndarray:
    """Raw matrix [rows][cols/block][block bytes] -> fp32 [rows][cols]
    (blocks of 256 weights for q2k/q4k/cb2, of 32 for q8)."""
    raw = np.asarray(raw, dtype=np.uint8)
    rows, nb = raw.shape[0], raw.shape[1]
    if fmt == "q2k":
        w = dequant_q2k(raw)
    elif fmt == "q4k":
        w = dequant_q4k(raw)
    elif fmt == "cb2":
        w = dequant_cb2(raw, codebook)
    elif fmt == "q8":
        return dequant_q8(raw).reshape(rows, nb * 32)
    else:
        raise ValueError(fmt)
    return w.reshape(rows, nb * 256)


# ---------------------------------------------------------------- router ---


def router_logits(x: np.ndarray, w_router: np.ndarray, bias=None) -> np.ndarray:
    """logit[t][e] = sum_h Wr[e][h] * x[t][h] + b[e], in fp64.  For fp32 x
    each product of two fp32 values is exact in fp64; x may also be an fp64
    vector (the pre-normalised input)."""
    lg = np.asarray(x, dtype=np.float64) @ np.asarray(w_router, dtype=np.float64).T
    if bias is not None:
        lg = lg + np.asarray(bias, dtype=np.float64)[None, :]
    return lg


def top_k(logits: np.ndarray, k: int):
    """Per token: the k experts with the largest logits, ranked by
    (logit descending, expert index ascending), and their weights.

    Weights: softmax over all experts followed by renormalisation over the
    selected k, which equals the softmax over the k selected logits:
    w_j = exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0), l_0 the largest.
    Also returns, per token, the gap between the k-th and (k+1)-th logit.
    """
    lg = np.asarray(logits, dtype=np.float64)
    T, E = lg.shape
    ids = np.empty((T, k), dtype=np.int32)
    wts = np.empty((T, k), dtype=np.float64)
    gap = np.full(T, np.inf)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-lg[t, e], e))
        sel = order[:k]
        ids[t] = sel
        z = np.exp(lg[t, sel] - lg[t, sel[0]])
        wts[t] = z / z.sum()
        if k < E:
            gap[t] = lg[t, order[k - 1]] - lg[t, order[k]]
    return ids, wts, gap


def group_by_expert(ids: np.ndarray, n_experts: int):
    """Stable bucket sort of the (token, slot) pairs by expert id.

    Returns counts[E], offsets[E+1], pairs (token * k + slot, ordered by
    expert, then token, then slot) and the ascending list of experts with a
    non-empty bucket.
    """
    ids = np.asarray(ids)
    T, k = ids.shape
    buckets = [[] for _ in range(n_experts)]
    for t in range(T):
        for j in range(k):
            buckets[int(ids[t, j])].append(t * k + j)
    counts = np.array([len(b) for b in buckets], dtype=np.int32)
    offsets = np.zeros(n_experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    pairs = np.array([p for b in buckets for p in b], dtype=np.int32)
    active = np.array([e for e in range(n_experts) if counts[e] > 0], dtype=np.int32)
    return counts, offsets, pairs, active


# ---------------------------------------------------------------- experts ---


def silu(v: np.ndarray) -> np.ndarray:
    """SiLU in fp64: v / (1 + exp(-v))."""
    return v / (1.0 + np.exp(-v))


def swiglu_ffn(x: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray):
    """One expert: a = silu(Wg x) * (Wu x); o = Wd a.  fp64 throughout.
    x [H]; wg, wu [F][H]; wd [H][F].  Returns (a [F], o [H])."""
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(wg, dtype=np.float64) @ x
    u = np.asarray(wu, dtype=np.float64) @ x
    a = silu(g) * u
    return a, np.asarray(wd, dtype=np.float64) @ a


class Layer:
    """One MoE layer's weights as the oracle reads them: the raw routed blocks
    plus dequantised matrices, cached per expert on first use."""

    def __init__(self, wl, lw, codebook):
        self.wl = wl
        self.lw = lw
        self.codebook = np.asarray(codebook)
        self._cache = {}
        self._slot = {e: i for i, e in enumerate(lw.experts)}

    def expert(self, e: int):
        if e not in self._cache:
            i = self._slot[e]
            wl, lw = self.wl, self.lw
            gfmt = getattr(lw, "gate_up_format", None) or wl.gate_up_format
            dfmt = getattr(lw, "down_format", None) or wl.down_format
            self._cache[e] = (
                dequant_matrix(lw.gate[i], gfmt, self.codebook),
                dequant_matrix(lw.up[i], gfmt, self.codebook),
                dequant_matrix(lw.down[i], dfmt, self.codebook),
            )
        return self._cache[e]

    def shared(self):
        if "shared" not in self._cache:
            lw = self.lw
            if getattr(self.wl, "shared_format", "bf16") == "q8":
                self._cache["shared"] = tuple(
                    dequant_matrix(m, "q8").astype(np.float64) for m in (lw.shared_gate, lw.shared_up, lw.shared_down))
            else:
                self._cache["shared"] = tuple(
                    bf16_bits_to_f64(m) for m in (lw.shared_gate, lw.shared_up, lw.shared_down))
        return self._cache["shared"]


RMS_EPS = 1e-6


def rms_inv(x: np.ndarray) -> np.ndarray:
    """Per row 1 / sqrt(mean(x^2) + eps) in fp64: the scale of an RMSNorm
    without learned weight, as the pre-norm residual stream of the pages'
    model families applies before each MoE block (norm layers are kept at
    f32 in the Quasar README, "Design decisions")."""
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / np.sqrt(np.mean(x * x, axis=-1) + RMS_EPS)


def route(lw, x: np.ndarray, k: int, prenorm: bool = False):
    """The routing of one layer for T tokens: the normalised input u (x, or
    x * rms_inv(x) with the pre-norm) is formed first and the router is
    evaluated on it.  Returns (u fp64 [T][H], logits, ids, w, gap)."""
    x = np.asarray(x, dtype=np.float32)
    u = x.astype(np.float64)
    if prenorm:
        u = u * rms_inv(x)[:, None]
    logits = router_logits(u, lw.router, lw.router_bias)
    ids, wts, gap = top_k(logits, k)
    return u, logits, ids, wts, gap


def steer(m: np.ndarray, direction: np.ndarray, scale: float) -> np.ndarray:
    """Directional steering of an FFN output (QuarkStar README, "Steering"):
    each row m becomes m - scale * d * (d . m), d the layer's direction taken
    as given (the pages store unit directions; nothing is normalised here).
    A positive scale removes the component along a unit d (scale 1 removes
    it entirely), a negative one amplifies it.  fp64."""
    m = np.asarray(m, dtype=np.float64)
    d = np.asarray(direction, dtype=np.float64)
    proj = m @ d                                   # d . m per row
    return m - scale * proj[..., None] * d


def moe_layer(layer: Layer, x: np.ndarray, residual: bool = False, prenorm: bool = False,
              steering=None):
    """One decode step of one MoE layer for T tokens.

    With u = x (or u = x * rms_inv(x) if prenorm):
    m[t] = sum_{j<k} w[t][j] * FFN_{ids[t][j]}(u[t]) + S(u[t]), with S the
    ungated shared expert (weight 1) when present and the router evaluated on
    u; with steering = (direction, scale) m is replaced by steer(m, ...);
    y[t] = m[t] (+ x[t] if residual).
    Returns a dict with y (fp32 [T][H]), ids, w (fp64), logits, gap.
    """
    wl, lw = layer.wl, layer.lw
    x = np.asarray(x, dtype=np.float32)
    T = x.shape[0]
    u, logits, ids, wts, gap = route(lw, x, wl.top_k, prenorm)
    y = np.zeros((T, wl.hidden), dtype=np.float64)
    for t in range(T):
        for j in range(wl.top_k):
            wg, wu, wd = layer.expert(int(ids[t, j]))
            _, o = swiglu_ffn(u[t], wg, wu, wd)
            y[t] += wts[t, j] * o
        if wl.shared_ffn:
            sg, su, sd = layer.shared()
            _, s = swiglu_ffn(u[t], sg, su, sd)
            y[t] += s
    if steering is not None:
        y = steer(y, steering[0], steering[1])
    if residual:
        y += x.astype(np.float64)
    return {"y": y.astype(np.float32), "ids": ids, "w": wts, "logits": logits, "gap": gap}


def moe_stack(layers, x: np.ndarray, prenorm: bool = True, steering=None):
    """Stacked layers chained by the residual stream:
    x_{l+1} = x_l + MoE_l(RMSNorm(x_l)) (pre-norm; without the norm an
    un-normalised SwiGLU chain grows without bound), each layer's output
    rounded to fp32.  steering = (directions [L][H], scale) steers every
    layer's MoE output with its own direction.  Returns the final x and the
    per-layer results."""
    outs = []
    cur = np.asarray(x, dtype=np.float32)
    for l, layer in enumerate(layers):
        st = None if steering is None else (steering[0][l], steering[1])
        r = moe_layer(layer, cur, residual=True, prenorm=prenorm, steering=st)
        outs.append(r)
        cur = r["y"]
    return cur, outs


def rel_l2(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per-row relative L2 error ||got - ref|| / ||ref|| in fp64."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.linalg.norm(got - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    return num / np.where(den == 0, 1.0, den)
