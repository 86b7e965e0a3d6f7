"""Test-side packers for hand-built quantized blocks.

These write the block formats in the packing direction (fields -> bytes), so a
decoder that reads a bit from the wrong place disagrees with the fields the
test chose.  Expected values are computed from those fields with exact
rational arithmetic, never by decoding.

q8_0 (34 bytes / 32 values): fp16 d, then 32 int8 codes; value = d*q.
q4_K (144 bytes / 256 values): fp16 d, fp16 dmin, 12 bytes holding eight 6-bit
scales sc[j] and eight 6-bit mins m[j], then 128 bytes of 4-bit codes; value
j*32+i of the block = d*sc[j]*q - dmin*m[j].  The 12 bytes: byte j (j<4) holds
sc[j] in bits 0-5 and the top two bits of sc[j+4] in bits 6-7; byte 4+j (j<4)
holds m[j] in bits 0-5 and the top two bits of m[j+4] in bits 6-7; byte 8+j
holds the low four bits of sc[j+4] (bits 0-3) and of m[j+4] (bits 4-7).  Code
byte 32*g+i holds value i of sub-block 2g (low nibble) and of sub-block 2g+1
(high nibble).
"""
from fractions import Fraction

import numpy as np


def half_bits(x: float) -> int:
    return int(np.array([x], dtype=np.float16).view(np.uint16)[0])


def half_value(bits: int) -> Fraction:
    """Exact value of an fp16 bit pattern, via numpy's conversion to float64."""
    v = np.array([bits], dtype=np.uint16).view(np.float16)[0]
    return Fraction(float(v))


def pack_q8_0(d_bits: int, q) -> bytes:
    q = [int(x) for x in q]
    assert len(q) == 32 and all(-128 <= x <= 127 for x in q)
    return bytes([d_bits & 0xFF, d_bits >> 8]) + bytes((x + 256) % 256 for x in q)


def q8_0_values(d_bits: int, q):
    d = half_value(d_bits)
    return [d * int(x) for x in q]


def pack_q4_K(d_bits: int, dmin_bits: int, sc, m, q) -> bytes:
    sc = [int(x) for x in sc]
    m = [int(x) for x in m]
    q = [int(x) for x in q]
    assert len(sc) == 8 and len(m) == 8 and len(q) == 256
    assert all(0 <= x < 64 for x in sc + m) and all(0 <= x < 16 for x in q)
    s = [0] * 12
    for j in range(4):
        s[j] = (sc[j] & 0x3F) | ((sc[j + 4] >> 4) << 6)
        s[4 + j] = (m[j] & 0x3F) | ((m[j + 4] >> 4) << 6)
        s[8 + j] = (sc[j + 4] & 0x0F) | ((m[j + 4] & 0x0F) << 4)
    qs = [0] * 128
    for g in range(4):
        for i in range(32):
            lo = q[64 * g + i]        # sub-block 2g, value i
            hi = q[64 * g + 32 + i]   # sub-block 2g+1, value i
            qs[32 * g + i] = lo | (hi << 4)
    head = bytes([d_bits & 0xFF, d_bits >> 8, dmin_bits & 0xFF, dmin_bits >> 8])
    return head + bytes(s) + bytes(qs)


def q4_K_values(d_bits: int, dmin_bits: int, sc, m, q):
    d = half_value(d_bits)
    dmin = half_value(dmin_bits)
    return [d * sc[e // 32] * int(q[e]) - dmin * m[e // 32] for e in range(256)]


def to_f32(values) -> np.ndarray:
    """Round exact rationals once to float32.  The values are multiples of 2^-24
    (or coarser) below 2^27, so float() is exact and the float32 cast is the
    only rounding."""
    return np.array([float(v) for v in values], dtype=np.float64).astype(np.float32)


# ---------------------------------------------------------------- the other GGUF types
# Layouts (GGUF block formats; multi-byte fields little-endian):
#   q4_0 (18 B / 32): fp16 d; code byte j holds value j (low nibble) and value
#     j+16 (high nibble); value = d*(q-8).
#   q4_1 (20 B / 32): fp16 d, fp16 m; codes as q4_0; value = d*q + m.
#   q5_0 (22 B / 32): fp16 d; 32-bit word whose bit j is bit 4 of value j;
#     nibbles as q4_0; value = d*(q-16).
#   q5_1 (24 B / 32): fp16 d, fp16 m; high-bit word; nibbles; value = d*q + m.
#   q2_K (84 B / 256): byte i (i < 16) = scale[i] | min[i] << 4 for the
#     sub-block of values 16i..16i+15; then 64 code bytes: value
#     128h + 32j + t sits in bits 2j..2j+1 of code byte 32h + t; fp16 d, fp16
#     dmin last; value = d*scale*q - dmin*min.
#   q3_K (110 B / 256): 32 mask bytes (bit 4h+j of mask byte t is set when
#     value 128h+32j+t is non-negative), 64 code bytes holding (q + 4) mod 4
#     at the q2_K positions, 12 scale bytes (6-bit s[i], stored biased by 32:
#     low nibble in byte i for i < 8 or the high nibble of byte i-8, top two
#     bits at bits 2*(i//4) of byte 8 + i%4), fp16 d; value = d*(s-32)*q.
#   q5_K (176 B / 256): fp16 d, fp16 dmin, 12 scale bytes packed as q4_K, 32
#     high-bit bytes (bit 2g+s of byte l is bit 4 of value 64g+32s+l), 128
#     nibble bytes as q4_K; value = d*sc*q - dmin*m.
#   q6_K (210 B / 256): 128 nibble bytes (value 128h+32c+l: nibble c//2 of
#     byte 64h + 32*(c%2) + l), 64 bytes of top bit pairs (bits 2c..2c+1 of
#     byte 32h + l), 16 int8 scales (sub-blocks of 16), fp16 d;
#     value = d*scale*(q-32) with q the 6-bit code.

def _u16(bits: int) -> bytes:
    return bytes([bits & 0xFF, (bits >> 8) & 0xFF])


def _nibbles32(q) -> bytes:
    return bytes((q[j] & 0x0F) | ((q[j + 16] & 0x0F) << 4) for j in range(16))


def _high32(q) -> bytes:
    w = 0
    for j in range(32):
        w |= ((q[j] >> 4) & 1) << j
    return w.to_bytes(4, "little")


def pack_q4_0(d_bits, q):
    assert len(q) == 32 and all(0 <= x < 16 for x in q)
    return _u16(d_bits) + _nibbles32(q)


def q4_0_values(d_bits, q):
    d = half_value(d_bits)
    return [d * (int(x) - 8) for x in q]


def pack_q4_1(d_bits, m_bits, q):
    assert len(q) == 32 and all(0 <= x < 16 for x in q)
    return _u16(d_bits) + _u16(m_bits) + _nibbles32(q)


def q4_1_values(d_bits, m_bits, q):
    d, m = half_value(d_bits), half_value(m_bits)
    return [d * int(x) + m for x in q]


def pack_q5_0(d_bits, q):
    assert len(q) == 32 and all(0 <= x < 32 for x in q)
    return _u16(d_bits) + _high32(q) + _nibbles32(q)


def q5_0_values(d_bits, q):
    d = half_value(d_bits)
    return [d * (int(x) - 16) for x in q]


def pack_q5_1(d_bits, m_bits, q):
    assert len(q) == 32 and all(0 <= x < 32 for x in q)
    return _u16(d_bits) + _u16(m_bits) + _high32(q) + _nibbles32(q)


def q5_1_values(d_bits, m_bits, q):
    d, m = half_value(d_bits), half_value(m_bits)
    return [d * int(x) + m for x in q]


def pack_q2_K(d_bits, dmin_bits, sc, mn, q):
    assert len(sc) == 16 and len(mn) == 16 and len(q) == 256
    assert all(0 <= x < 16 for x in list(sc) + list(mn)) and all(0 <= x < 4 for x in q)
    scales = bytes(int(sc[i]) | (int(mn[i]) << 4) for i in range(16))
    codes = [0] * 64
    for h in range(2):
        for j in range(4):
            for t in range(32):
                codes[32 * h + t] |= int(q[128 * h + 32 * j + t]) << (2 * j)
    return scales + bytes(codes) + _u16(d_bits) + _u16(dmin_bits)


def q2_K_values(d_bits, dmin_bits, sc, mn, q):
    d, dmin = half_value(d_bits), half_value(dmin_bits)
    return [d * int(sc[v // 16]) * int(q[v]) - dmin * int(mn[v // 16]) for v in range(256)]


def pack_q3_K(d_bits, s6, q):
    """s6: the 16 stored 6-bit scales (0..63, value s6 - 32); q in -4..3."""
    assert len(s6) == 16 and len(q) == 256
    assert all(0 <= x < 64 for x in s6) and all(-4 <= x < 4 for x in q)
    mask = [0] * 32
    codes = [0] * 64
    for h in range(2):
        for j in range(4):
            for t in range(32):
                x = int(q[128 * h + 32 * j + t])
                if x >= 0:
                    mask[t] |= 1 << (4 * h + j)
                codes[32 * h + t] |= ((x + 4) & 3) << (2 * j)
    sb = [0] * 12
    for i in range(16):
        lo, hi = int(s6[i]) & 0x0F, int(s6[i]) >> 4
        if i < 8:
            sb[i] |= lo
        else:
            sb[i - 8] |= lo << 4
        sb[8 + i % 4] |= hi << (2 * (i // 4))
    return bytes(mask) + bytes(codes) + bytes(sb) + _u16(d_bits)


def q3_K_values(d_bits, s6, q):
    d = half_value(d_bits)
    return [d * (int(s6[v // 16]) - 32) * int(q[v]) for v in range(256)]


def _q4k_scale_bytes(sc, m):
    s = [0] * 12
    for j in range(4):
        s[j] = (sc[j] & 0x3F) | ((sc[j + 4] >> 4) << 6)
        s[4 + j] = (m[j] & 0x3F) | ((m[j + 4] >> 4) << 6)
        s[8 + j] = (sc[j + 4] & 0x0F) | ((m[j + 4] & 0x0F) << 4)
    return bytes(s)


def pack_q5_K(d_bits, dmin_bits, sc, m, q):
    sc = [int(x) for x in sc]
    m = [int(x) for x in m]
    assert len(sc) == 8 and len(m) == 8 and len(q) == 256
    assert all(0 <= x < 64 for x in sc + m) and all(0 <= x < 32 for x in q)
    high = [0] * 32
    qs = [0] * 128
    for g in range(4):
        for s in range(2):
            for l in range(32):
                x = int(q[64 * g + 32 * s + l])
                qs[32 * g + l] |= (x & 0x0F) << (4 * s)
                high[l] |= (x >> 4) << (2 * g + s)
    return _u16(d_bits) + _u16(dmin_bits) + _q4k_scale_bytes(sc, m) + bytes(high) + bytes(qs)


def q5_K_values(d_bits, dmin_bits, sc, m, q):
    d, dmin = half_value(d_bits), half_value(dmin_bits)
    return [d * int(sc[v // 32]) * int(q[v]) - dmin * int(m[v // 32]) for v in range(256)]


def pack_q6_K(d_bits, sc, q):
    """sc: 16 int8 scales; q: 256 values in -32..31 (stored as q + 32)."""
    assert len(sc) == 16 and len(q) == 256
    assert all(-128 <= x < 128 for x in sc) and all(-32 <= x < 32 for x in q)
    ql = [0] * 128
    qh = [0] * 64
    for h in range(2):
        for c in range(4):
            for l in range(32):
                u = int(q[128 * h + 32 * c + l]) + 32
                ql[64 * h + 32 * (c % 2) + l] |= (u & 0x0F) << (4 * (c // 2))
                qh[32 * h + l] |= (u >> 4) << (2 * c)
    return bytes(ql) + bytes(qh) + bytes((int(x) + 256) % 256 for x in sc) + _u16(d_bits)


def q6_K_values(d_bits, sc, q):
    d = half_value(d_bits)
    return [d * int(sc[v // 16]) * int(q[v]) for v in range(256)]
