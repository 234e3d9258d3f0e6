"""Pins of the oracle's scalar decoders and block dequantisation.

The oracle is checked against things other than itself: library routines
for the fp16/bf16 decoders, hand-worked block values (tests/golden), and
locality / linearity invariants of the two block layouts that a misplaced
nibble, bit or byte would break.
"""
import os

import numpy as np
import pytest
import torch

from oracle import moe as om

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "handworked_blocks.txt")


# ------------------------------------------------------- block packers ---
# Independent encoders: field values -> raw block bytes, following the layout
# tables (they share nothing with the oracle's decoders).

def pack_q2k(d=0, dmin=0, sc=None, m=None, q=None):
    blk = np.zeros(84, dtype=np.uint8)
    sc = np.zeros(16, int) if sc is None else np.asarray(sc)
    m = np.zeros(16, int) if m is None else np.asarray(m)
    q = np.zeros(256, int) if q is None else np.asarray(q)
    for i in range(16):
        blk[i] = (int(sc[i]) & 15) | ((int(m[i]) & 15) << 4)
    for byte in range(64):
        v = 0
        for p in range(4):
            v |= (int(q[4 * byte + p]) & 3) << (2 * p)
        blk[16 + byte] = v
    blk[80], blk[81] = d & 0xFF, d >> 8
    blk[82], blk[83] = dmin & 0xFF, dmin >> 8
    return blk


def pack_cb2(d=0, s=None, idx=None, sign=None):
    blk = np.zeros(70, dtype=np.uint8)
    s = np.zeros(8, int) if s is None else np.asarray(s)
    idx = np.zeros(32, int) if idx is None else np.asarray(idx)
    sign = np.zeros(32, int) if sign is None else np.asarray(sign)
    blk[0], blk[1] = d & 0xFF, d >> 8
    for i in range(8):
        blk[2 + i // 2] |= (int(s[i]) & 15) << (4 * (i % 2))
    blk[6:38] = idx
    blk[38:70] = sign
    return blk


def pack_q8(d=0, q=None):
    blk = np.zeros(34, dtype=np.uint8)
    q = np.zeros(32, int) if q is None else np.asarray(q)
    blk[0], blk[1] = d & 0xFF, d >> 8
    blk[2:34] = (q.astype(np.int64) & 0xFF).astype(np.uint8)
    return blk


def hand_codebook():
    cb = np.ones((256, 8), dtype=np.int8)
    cb[7] = [1, 3, 5, 7, 7, 5, 3, 1]
    return cb


# ----------------------------------------------------------- decoders ---

def test_fp16_decode_matches_numpy_all_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    got = om.fp16_bits_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zero kept
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def test_bf16_decode_matches_torch_all_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    got = om.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# ------------------------------------------------- hand-worked fixtures ---

def _parse_golden():
    cases = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            fmt, fields, j, expected, _why = [c.strip() for c in line.split("|")]
            kv = {}
            for tok in fields.split():
                k, v = tok.split("=")
                kv[k] = v
            cases.append((fmt, kv, int(j), float(expected), line))
    return cases


def _indexed(kv, name, n, base=10):
    out = np.zeros(n, int)
    for k, v in kv.items():
        if k.startswith(name) and k[len(name):].isdigit():
            out[int(k[len(name):])] = int(v, base)
    return out


@pytest.mark.parametrize("case", _parse_golden(), ids=lambda c: c[4][:60])
def test_handworked_block(case):
    fmt, kv, j, expected, _ = case
    if fmt == "q2k":
        blk = pack_q2k(d=int(kv.get("d", "0"), 16), dmin=int(kv.get("dmin", "0"), 16),
                       sc=_indexed(kv, "sc", 16), m=_indexed(kv, "m", 16), q=_indexed(kv, "q", 256))
        w = om.dequant_q2k(blk)
    elif fmt == "q8":
        blk = pack_q8(d=int(kv.get("d", "0"), 16), q=_indexed(kv, "q", 32))
        w = om.dequant_q8(blk)
    elif fmt == "q4k":
        # raw bytes, no encoder: the byte offsets themselves are what is pinned
        blk = np.zeros(144, dtype=np.uint8)
        for name, off in (("d", 0), ("dmin", 2)):
            v = int(kv.get(name, "0"), 16)
            blk[off], blk[off + 1] = v & 0xFF, v >> 8
        raw = _indexed(kv, "b", 144, 16)
        blk[4:] = raw[4:]
        w = om.dequant_q4k(blk)
    else:
        blk = pack_cb2(d=int(kv.get("d", "0"), 16), s=_indexed(kv, "s", 8),
                       idx=_indexed(kv, "idx", 32), sign=_indexed(kv, "sign", 32, 16))
        w = om.dequant_cb2(blk, hand_codebook())
    assert w.dtype == np.float32
    assert w[j] == np.float32(expected)
    if expected == 0.0 and str(expected).startswith("-"):
        assert np.signbit(w[j])


def test_golden_file_has_cases():
    cases = _parse_golden()
    assert sum(c[0] == "q2k" for c in cases) >= 8 and sum(c[0] == "cb2" for c in cases) >= 8
    assert sum(c[0] == "q8" for c in cases) >= 6
    assert sum(c[0] == "q4k" for c in cases) >= 8


# ---------------------------------------------------- layout invariants ---

RNG = np.random.default_rng(1234)


def _rand_q2k():
    return pack_q2k(d=int(RNG.integers(0x0400, 0x3C00)), dmin=int(RNG.integers(0x0400, 0x3C00)),
                    sc=RNG.integers(0, 16, 16), m=RNG.integers(0, 16, 16), q=RNG.integers(0, 4, 256))


def test_q2k_each_code_moves_only_its_weight():
    """Changing the 2-bit code at qs byte b, bits 2p..2p+1 changes exactly
    weight 4b+p, by d*sc*(delta q) (exact)."""
    blk = _rand_q2k()
    d = om.fp16_bits_to_f64(int(blk[80]) | int(blk[81]) << 8)
    base = om.dequant_q2k(blk).astype(np.float64)
    for b in range(0, 64, 7):
        for p in range(4):
            blk2 = blk.copy()
            old = (int(blk2[16 + b]) >> (2 * p)) & 3
            new = (old + 1) & 3
            blk2[16 + b] = (int(blk2[16 + b]) & ~(3 << (2 * p)) & 0xFF) | (new << (2 * p))
            w2 = om.dequant_q2k(blk2).astype(np.float64)
            changed = np.nonzero(w2 != base)[0]
            j = 4 * b + p
            sc = int(blk[(j // 16)]) & 15
            if sc == 0:
                assert changed.size == 0
                continue
            assert list(changed) == [j]
            # both values are d*sc*q - dmin*m rounded once; compare the exact part
            dmin = om.fp16_bits_to_f64(int(blk[82]) | int(blk[83]) << 8)
            m = int(blk[j // 16]) >> 4
            assert w2[j] == np.float32(d * sc * new - dmin * m)


def test_q2k_scale_nibbles():
    """Low nibble of scales[i] scales the codes of sub-block i only; the high
    nibble is the min of sub-block i only."""
    q = np.full(256, 2)
    for i in range(16):
        sc = np.zeros(16, int)
        sc[i] = 5
        w = om.dequant_q2k(pack_q2k(d=0x3C00, sc=sc, q=q))
        expect = np.zeros(256, np.float32)
        expect[16 * i:16 * i + 16] = 10.0
        assert np.array_equal(w, expect)
        m = np.zeros(16, int)
        m[i] = 3
        w = om.dequant_q2k(pack_q2k(dmin=0x3800, m=m, q=q))
        expect = np.zeros(256, np.float32)
        expect[16 * i:16 * i + 16] = -1.5
        assert np.array_equal(w, expect)


def test_q2k_d_and_dmin_positions():
    sc = np.ones(16, int)
    m = np.ones(16, int)
    q = np.ones(256, int)
    assert np.all(om.dequant_q2k(pack_q2k(d=0x4000, sc=sc, m=m, q=q)) == 2.0)
    assert np.all(om.dequant_q2k(pack_q2k(dmin=0x4000, sc=sc, m=m, q=q)) == -2.0)


def test_cb2_sign_bits_and_groups():
    """Bit b of sign[g] negates weight 8g+b only; idx[g] picks the row for
    weights 8g..8g+7 only."""
    cb = synth_codebook()
    base_idx = RNG.integers(0, 256, 32)
    s = RNG.integers(1, 16, 8)
    blk = pack_cb2(d=0x3C00, s=s, idx=base_idx)
    w0 = om.dequant_cb2(blk, cb)
    assert np.all(w0 > 0)
    for g in range(0, 32, 5):
        for b in range(8):
            sign = np.zeros(32, int)
            sign[g] = 1 << b
            w = om.dequant_cb2(pack_cb2(d=0x3C00, s=s, idx=base_idx, sign=sign), cb)
            diff = np.nonzero(w != w0)[0]
            assert list(diff) == [8 * g + b]
            assert w[8 * g + b] == -w0[8 * g + b]
        idx2 = base_idx.copy()
        idx2[g] = (idx2[g] + 1) % 256
        w = om.dequant_cb2(pack_cb2(d=0x3C00, s=s, idx=idx2), cb)
        j = np.arange(256)
        outside = (j // 8) != g
        assert np.array_equal(w[outside], w0[outside])
        i = (8 * g) // 32
        assert np.array_equal(w[8 * g:8 * g + 8], (s[i] * cb[idx2[g]]).astype(np.float32))


def test_cb2_scale_nibbles_and_d():
    cb = np.ones((256, 8), dtype=np.int8)
    for i in range(8):
        s = np.zeros(8, int)
        s[i] = 3
        w = om.dequant_cb2(pack_cb2(d=0x3800, s=s), cb)
        expect = np.zeros(256, np.float32)
        expect[32 * i:32 * i + 32] = 1.5
        assert np.array_equal(w, expect)


def test_exact_linearity_in_d():
    """Doubling d (exactly, via the fp16 exponent) doubles every codebook
    weight and every d*sc*q term exactly."""
    cb = synth_codebook()
    s = RNG.integers(0, 16, 8)
    idx = RNG.integers(0, 256, 32)
    sign = RNG.integers(0, 256, 32)
    w1 = om.dequant_cb2(pack_cb2(d=0x3555, s=s, idx=idx, sign=sign), cb)
    w2 = om.dequant_cb2(pack_cb2(d=0x3555 + 0x0400, s=s, idx=idx, sign=sign), cb)
    assert np.array_equal(w2, 2 * w1)
    sc = RNG.integers(0, 16, 16)
    q = RNG.integers(0, 4, 256)
    a = om.dequant_q2k(pack_q2k(d=0x3555, sc=sc, q=q))
    b = om.dequant_q2k(pack_q2k(d=0x3955, sc=sc, q=q))
    assert np.array_equal(b, 2 * a)


def test_exhaustive_q2k_fields_single_rounding():
    """All (sc, m, q) combinations: the value is the exact d*sc*q - dmin*m
    (computed here with integer arithmetic on the fp16 significands) rounded
    once to fp32."""
    from fractions import Fraction
    d_bits, dmin_bits = 0x2A5B, 0x1C37          # two normal fp16 values
    dF = Fraction(float(om.fp16_bits_to_f64(d_bits)))
    dmF = Fraction(float(om.fp16_bits_to_f64(dmin_bits)))
    combos = [(sc, m) for sc in range(16) for m in range(16)]
    for start in range(0, len(combos), 16):
        chunk = combos[start:start + 16]
        sc = [c[0] for c in chunk]
        m = [c[1] for c in chunk]
        q = np.tile(np.arange(4).repeat(4), 16)
        w = om.dequant_q2k(pack_q2k(d=d_bits, dmin=dmin_bits, sc=sc, m=m, q=q))
        for j in range(256):
            i = j // 16
            exact = dF * sc[i] * int(q[j]) - dmF * m[i]
            assert w[j] == np.float32(float(exact)), (sc[i], m[i], q[j])


def test_exhaustive_cb2_index_and_sign_bytes():
    """Every (idx byte, sign byte) pair: 65536 groups over 2048 blocks."""
    cb = synth_codebook()
    pairs = np.arange(65536)
    idx_all = pairs // 256
    sign_all = pairs % 256
    s = np.array([1, 2, 3, 4, 5, 6, 7, 15])
    blocks = np.stack([pack_cb2(d=0x3C00, s=s, idx=idx_all[32 * b:32 * b + 32],
                                sign=sign_all[32 * b:32 * b + 32]) for b in range(2048)])
    w = om.dequant_cb2(blocks, cb).reshape(2048, 32, 8)
    j = np.arange(256).reshape(32, 8)
    sub = s[j // 32]                                        # [32][8]
    mag = cb[idx_all.reshape(2048, 32)].astype(np.int64) * sub[None]  # [2048][32][8]
    neg = (sign_all.reshape(2048, 32)[:, :, None] >> np.arange(8)) & 1
    expect = np.where(neg == 1, -mag, mag).astype(np.float32)
    assert np.array_equal(w, expect)


def synth_codebook():
    import synth
    return synth.codebook()


def test_codebook_entries():
    cb = synth_codebook()
    assert cb.shape == (256, 8) and cb.dtype == np.int8
    assert set(np.unique(cb)) == {1, 3, 5, 7}


# ------------------------------------------------- matrix block order ---

def _fp16_bits(v):
    return int(np.array([v], dtype=np.float16).view(np.uint16)[0])


@pytest.mark.parametrize("fmt", ["q2k", "cb2", "q8", "q4k"])
def test_dequant_matrix_block_order(fmt):
    """A matrix is [rows][cols/256] blocks, row-major: block (r, b) holds
    columns 256*b .. 256*b+255 of row r.  Every block here decodes to the
    constant r*nb + b + 1 (its d, with unit scale and code), so a transposed
    or shuffled block order shows up as a wrong constant."""
    rows, nb = 3, 4
    raw = []
    for r in range(rows):
        row = []
        for b in range(nb):
            d = _fp16_bits(float(r * nb + b + 1))
            if fmt == "q2k":   # w = d*1*1 - 0*0
                row.append(pack_q2k(d=d, sc=np.ones(16, int), q=np.ones(256, int)))
            elif fmt == "cb2":  # w = d*1*C[0][j%8] with an all-ones codebook row 0
                row.append(pack_cb2(d=d, s=np.ones(8, int)))
            elif fmt == "q4k":  # every sc = 1 (bytes 4..7 and the low nibbles of 12..15), m = 0, codes 1
                blk = np.zeros(144, dtype=np.uint8)
                blk[0], blk[1] = d & 0xFF, d >> 8
                blk[4:8] = 1
                blk[12:16] = 1
                blk[16:144] = 0x11
                row.append(blk)
            else:              # w = d*1
                row.append(pack_q8(d=d, q=np.ones(32, int)))
        raw.append(row)
    raw = np.array(raw, dtype=np.uint8)
    bw = 32 if fmt == "q8" else 256
    w = om.dequant_matrix(raw, fmt, hand_codebook())
    assert w.shape == (rows, nb * bw)
    for r in range(rows):
        for b in range(nb):
            assert np.all(w[r, bw * b:bw * (b + 1)] == np.float32(r * nb + b + 1)), (r, b)


def _rand_q4k(rng):
    blk = rng.integers(0, 256, 144).astype(np.uint8)
    for off in (0, 2):   # normal fp16 d and dmin
        v = _fp16_bits(float(rng.uniform(0.25, 2.0)))
        blk[off], blk[off + 1] = v & 0xFF, v >> 8
    return blk


def test_q4k_each_code_nibble_moves_only_its_weight():
    rng = np.random.default_rng(41)
    for _ in range(4):
        blk = _rand_q4k(rng)
        w0 = om.dequant_q4k(blk)
        for byte in range(128):
            c, r = byte // 32, byte % 32
            for hi in (0, 1):
                b2 = blk.copy()
                b2[16 + byte] ^= 0xF0 if hi else 0x0F
                moved = np.nonzero(om.dequant_q4k(b2) != w0)[0]
                want = 64 * c + r + 32 * hi
                assert set(moved) <= {want}, (byte, hi, moved)


def test_q4k_each_scale_byte_moves_only_its_sub_blocks():
    """Byte 4+j (j < 4) holds sc of sub-block j (low 6 bits) and the top bits
    of sc of sub-block j+4; byte 8+j holds m of j and the top bits of m of
    j+4; byte 12+j holds the low nibbles of sc and m of sub-block j+4."""
    rng = np.random.default_rng(42)
    owners = {}
    for j in range(4):
        owners[4 + j] = {j, j + 4}
        owners[8 + j] = {j, j + 4}
        owners[12 + j] = {j + 4}
    for _ in range(4):
        blk = _rand_q4k(rng)
        blk[16:144] = 0x77   # every code 7: every sub-block shows its sc
        w0 = om.dequant_q4k(blk)
        for byte, subs in owners.items():
            for bit in range(8):
                b2 = blk.copy()
                b2[byte] ^= 1 << bit
                moved = set(np.nonzero(om.dequant_q4k(b2) != w0)[0] // 32)
                assert moved and moved <= subs, (byte, bit, moved)
                low6 = byte < 12 and bit < 6
                if low6:      # the low 6 bits belong to sub-block byte%4 only
                    assert moved == {(byte - 4) % 4}, (byte, bit, moved)


def test_q4k_exact_linearity_in_d_and_dmin():
    rng = np.random.default_rng(43)
    for _ in range(8):
        blk = _rand_q4k(rng)
        w = om.dequant_q4k(blk).astype(np.float64)
        b2 = blk.copy()
        for off in (0, 2):   # exponent + 1: exactly twice the value (normal fp16)
            v = (int(b2[off]) | int(b2[off + 1]) << 8) + 0x0400
            b2[off], b2[off + 1] = v & 0xFF, v >> 8
        assert np.array_equal(om.dequant_q4k(b2).astype(np.float64), 2 * w)


def test_q8_code_bytes_are_signed_and_linear():
    """Every code byte 0..255 read as a signed int8 (0x80 = -128, 0xFF = -1);
    each weight moves only with its own byte, exactly linearly."""
    d = _fp16_bits(0.25)
    for start in range(0, 256, 32):
        codes = np.arange(start, start + 32)
        blk = pack_q8(d=d)
        blk[2:34] = codes.astype(np.uint8)
        w = om.dequant_q8(blk)
        signed = np.where(codes >= 128, codes - 256, codes)
        assert np.all(w == np.float32(0.25) * signed.astype(np.float32))
