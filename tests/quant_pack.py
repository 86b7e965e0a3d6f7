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
