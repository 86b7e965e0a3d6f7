// block_formats.h -- device decoders of the frozen-weight block types, one
// group of 8 consecutive values of a row at a time.
//
// The types are the ones OUT_PROD reads for a (pages: the MUL_MAT_ID_BACK
// page lists them as out_prod's set: f16, bf16, q4_0, q4_1, q5_0, q5_1,
// q8_0, q2_K..q6_K); the byte layouts are the GGUF block formats as publicly
// documented (little-endian fields).  q8_0 and q4_K have loaders of their
// own in the tiled kernel; this header covers the others.
//
// A format F provides
//   QK, BYTES   values and bytes per block
//   NW          32-bit registers that hold one group's raw bits
//   fetch(blk, w, r)   global loads of what values w..w+7 of block `blk` need
//                      (w a multiple of 8), issued a pipeline stage early
//   decode(r, w, v)    the 8 values as fp32
// Blocks whose size is a multiple of 4 are read with 32-bit loads, the others
// (2-byte aligned) with 16-bit loads.  A group of registers left at zero
// decodes to zeros (every format's values carry a factor d).
//
// Exactness: each value is the block formula's exact result rounded once to
// fp32.  Products of an fp16 scale (11 significant bits) with the 4-8 bit
// sub-block scales and codes are exact in fp32; only q4_1/q5_1's "+ m", the
// K-quants' "- dmin*min" and q6_K's 25-bit d*scale*q round, once.
#pragma once

#include <stdint.h>

#include "kernel_common.h"

namespace outprod {

__device__ __forceinline__ uint32_t ld_u16(const uint8_t *p) { return *(const uint16_t *)p; }
__device__ __forceinline__ uint32_t ld_u32(const uint8_t *p) { return *(const uint32_t *)p; }
// 4 bytes from a 2-byte aligned address
__device__ __forceinline__ uint32_t ld_u32_a2(const uint8_t *p) {
    return ld_u16(p) | (ld_u16(p + 2) << 16);
}
__device__ __forceinline__ uint32_t byte_of(uint32_t lo, uint32_t hi, int e) {
    return ((e < 4 ? lo : hi) >> (8 * (e & 3))) & 0xFFu;
}
// byte e of a dword as float (one v_cvt_f32_ubyte)
__device__ __forceinline__ float ubyte(uint32_t w, int e) { return (float)((w >> (8 * e)) & 0xFFu); }
// bits 0-3 of x moved to bit 0 of bytes 0-3 (the four partial products do
// not overlap, so the multiply has no carries into the kept bits)
__device__ __forceinline__ uint32_t spread4(uint32_t x) { return ((x & 0xFu) * 0x00204081u) & 0x01010101u; }

// q4_0: fp16 d; 16 code bytes -- byte j holds value j (low nibble) and value
// j+16 (high nibble); value = d*(q - 8).
struct FmtQ4_0 {
    static constexpr int QK = 32, BYTES = 18, NW = 3;
    __device__ static void fetch(const uint8_t *blk, int w, uint32_t (&r)[NW]) {
        r[0] = ld_u16(blk);
        r[1] = ld_u32_a2(blk + 2 + (w & 15));
        r[2] = ld_u32_a2(blk + 6 + (w & 15));
    }
    __device__ static void decode(const uint32_t (&r)[NW], int w, float (&v)[8]) {
        const float d = half_bits_to_float(r[0]), off = -8.f * d;  // exact
        const int sh = w >= 16 ? 4 : 0;
        const uint32_t n0 = opaque((r[1] >> sh) & 0x0F0F0F0Fu), n1 = opaque((r[2] >> sh) & 0x0F0F0F0Fu);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // d*q - 8d = d*(q - 8): exact (<= 15 significant bits)
            v[e] = __builtin_fmaf(d, ubyte(n0, e), off);
            v[4 + e] = __builtin_fmaf(d, ubyte(n1, e), off);
        }
    }
};

// q4_1: fp16 d, fp16 m; codes as q4_0; value = d*q + m.
struct FmtQ4_1 {
    static constexpr int QK = 32, BYTES = 20, NW = 3;
    __device__ static void fetch(const uint8_t *blk, int w, uint32_t (&r)[NW]) {
        r[0] = ld_u32(blk);
        r[1] = ld_u32(blk + 4 + (w & 15));
        r[2] = ld_u32(blk + 8 + (w & 15));
    }
    __device__ static void decode(const uint32_t (&r)[NW], int w, float (&v)[8]) {
        const float d = half_bits_to_float(r[0] & 0xFFFFu), m = half_bits_to_float(r[0] >> 16);
        const int sh = w >= 16 ? 4 : 0;
        const uint32_t n0 = opaque((r[1] >> sh) & 0x0F0F0F0Fu), n1 = opaque((r[2] >> sh) & 0x0F0F0F0Fu);
#pragma unroll
        for (int e = 0; e < 4; ++e) {  // d*q exact, one rounding with + m
            v[e] = __builtin_fmaf(d, ubyte(n0, e), m);
            v[4 + e] = __builtin_fmaf(d, ubyte(n1, e), m);
        }
    }
};

// q5_0: fp16 d; 32-bit word whose bit j is bit 4 of value j; low nibbles as
// q4_0; value = d*(q - 16).
struct FmtQ5_0 {
    static constexpr int QK = 32, BYTES = 22, NW = 4;
    __device__ static void fetch(const uint8_t *blk, int w, uint32_t (&r)[NW]) {
        r[0] = ld_u16(blk);
        r[1] = ld_u16(blk + 2 + 2 * (w >> 4));  // high-bit bytes w/8 (and its neighbour)
        r[2] = ld_u32_a2(blk + 6 + (w & 15));
        r[3] = ld_u32_a2(blk + 10 + (w & 15));
    }
    __device__ static void decode(const uint32_t (&r)[NW], int w, float (&v)[8]) {
        const float d = half_bits_to_float(r[0]), off = -16.f * d;  // exact
        const int sh = w >= 16 ? 4 : 0;
        const uint32_t hb = (r[1] >> (8 * ((w >> 3) & 1))) & 0xFFu;
        const uint32_t n0 = opaque(((r[2] >> sh) & 0x0F0F0F0Fu) | (spread4(hb) << 4));
        const uint32_t n1 = opaque(((r[3] >> sh) & 0x0F0F0F0Fu) | (spread4(hb >> 4) << 4));
#pragma unroll
        for (int e = 0; e < 4; ++e) {  // d*(q - 16): exact
            v[e] = __builtin_fmaf(d, ubyte(n0, e), off);
            v[4 + e] = __builtin_fmaf(d, ubyte(n1, e), off);
        }
    }
};

// q5_1: fp16 d, fp16 m; high-bit word; low nibbles; value = d*q + m.
struct FmtQ5_1 {
    static constexpr int QK = 32, BYTES = 24, NW = 4;
    __device__ static void fetch(const uint8_t *blk, int w, uint32_t (&r)[NW]) {
        r[0] = ld_u32(blk);
        r[1] = ld_u32(blk + 4);
        r[2] = ld_u32(blk + 8 + (w & 15));
        r[3] = ld_u32(blk + 12 + (w & 15));
    }
    __device__ static void decode(const uint32_t (&r)[NW], int w, float (&v)[8]) {
        const float d = half_bits_to_float(r[0] & 0xFFFFu), m = half_bits_to_float(r[0] >> 16);
        const int sh = w >= 16 ? 4 : 0;
        const uint32_t hb = (r[1] >> w) & 0xFFu;
        const uint32_t n0 = opaque(((r[2] >> sh) & 0x0F0F0F0Fu) | (spread4(hb) << 4));
        const uint32_t n1 = opaque(((r[3] >> sh) & 0x0F0F0F0Fu) | (spread4(hb >> 4) << 4));
#pragma unroll
        for (int e = 0; e < 4; ++e) {  // d*q exact, one rounding with + m
            v[e] = __builtin_fmaf(d, ubyte(n0, e), m);
            v[4 + e] = __builtin_fmaf(d, ubyte(n1, e), m);
        }
    }
};

// q2_K: 16 bytes (scale | min << 4) for sub-blocks of 16 values; 64 code
// bytes (value 128h + 32j + t: bits 2j..2j+1 of byte 32h + t); fp16 d, fp16
// dmin at 80.  value = d*scale*q - dmin*min.
struct FmtQ2_K {
    static constexpr int QK = 256, BYTES = 84, NW = 4;
    __device__ static void fetch(const uint8_t *blk, int w, uint32_t (&r)[NW]) {
        const int h = w >> 7, t0 = w & 31;
        r[0] = ld_u32(blk + 80);
        r[1] = ld_u32(blk + 4 * (w >> 6));  // holds scale byte w/16
        r[2] = ld_u32(blk + 16 + 32 * h + t0);
        r[3] = ld_u32(blk + 20 + 32 * h + t0);
    }
    __device__ static void decode(const uint32_t (&r)[NW], int w, float (&v)[8]) {
        const float d = half_bits_to_float(r[0] & 0xFFFFu), dmin = half_bits_to_float(r[0] >> 16);
        const uint32_t sm = (r[1] >> (8 * ((w >> 4) & 3))) & 0xFFu;
        const float ds = d * (float)(sm & 0xFu), dm = dmin * (float)(sm >> 4);
        const int sh = 2 * ((w >> 5) & 3);
        const uint32_t n0 = opaque((r[2] >> sh) & 0x03030303u), n1 = opaque((r[3] >> sh) & 0x03030303u);
#pragma unroll
        for (int e = 0; e < 4; ++e) {  // ds*q exact, one rounding with - dm
            v[e] = __builtin_fmaf(ds, ubyte(n0, e), -dm);
            v[4 + e] = __builtin_fmaf(ds, ubyte(n1, e), -dm);
        }
    }
};

// q3_K: 32 mask bytes (bit 4h+j of byte t set: value 128h+32j+t keeps its
// low two bits, else they are lowered by 4), 64 code bytes at 32 (q2_K's
// positions), 12 bytes of 6-bit scales at 96 (low nibble in byte i or the
// high nibble of byte i-8; top bits at 2*(i/4) of byte 8+i%4; biased by 32),
// fp16 d at 108.  value = d*(scale-32)*q, exact.
struct FmtQ3_K {
    static constexpr int QK = 256, BYTES = 110, NW = 7;
    __device__ static void fetch(const uint8_t *blk, int w, uint32_t (&r)[NW]) {
        const int h = w >> 7, t0 = w & 31, i = w >> 4;
        r[0] = ld_u16(blk + 108);
        r[1] = ld_u32_a2(blk + t0);
        r[2] = ld_u32_a2(blk + t0 + 4);
        r[3] = ld_u32_a2(blk + 32 + 32 * h + t0);
        r[4] = ld_u32_a2(blk + 36 + 32 * h + t0);
        r[5] = ld_u16(blk + 96 + 2 * ((i & 7) >> 1));       // low-nibble byte i%8
        r[6] = ld_u16(blk + 104 + 2 * ((i & 3) >> 1));      // top-bits byte 8 + i%4
    }
    __device__ static void decode(const uint32_t (&r)[NW], int w, float (&v)[8]) {
        const int h = w >> 7, j = (w >> 5) & 3, i = w >> 4;
        const uint32_t lob = (r[5] >> (8 * (i & 1))) & 0xFFu;
        const uint32_t hib = (r[6] >> (8 * (i & 1))) & 0xFFu;
        const uint32_t lo4 = i < 8 ? (lob & 0xFu) : (lob >> 4);
        const uint32_t hi2 = (hib >> (2 * (i >> 2))) & 3u;
        const float dl = half_bits_to_float(r[0]) * (float)((int)(lo4 | (hi2 << 4)) - 32);
        const int hs = 4 * h + j;
        // u = low | keep << 2 in each byte; q = u - 4 (keep set: q = low)
        const uint32_t u0 = opaque(((r[3] >> (2 * j)) & 0x03030303u) | (((r[1] >> hs) & 0x01010101u) << 2));
        const uint32_t u1 = opaque(((r[4] >> (2 * j)) & 0x03030303u) | (((r[2] >> hs) & 0x01010101u) << 2));
        const float off = -4.f * dl;  // exact
#pragma unroll
        for (int e = 0; e < 4; ++e) {  // dl*(u - 4): exact
            v[e] = __builtin_fmaf(dl, ubyte(u0, e), off);
            v[4 + e] = __builtin_fmaf(dl, ubyte(u1, e), off);
        }
    }
};

// 6-bit scale and min of sub-block `sub` (0..7) from the 12 packed bytes of
// q4_K / q5_K (bytes 0-3 in s0, 4-7 in s1, 8-11 in s2): for sub < 4 the low
// 6 bits of bytes sub and 4+sub; otherwise the nibbles of byte 8+(sub-4)
// below the top two bits of bytes sub-4 and sub.
__device__ __forceinline__ void k4_scale_min(uint32_t s0, uint32_t s1, uint32_t s2, int sub,
                                             uint32_t *sc, uint32_t *mn) {
    if (sub < 4) {
        *sc = (s0 >> (8 * sub)) & 0x3Fu;
        *mn = (s1 >> (8 * sub)) & 0x3Fu;
    } else {
        const int sh = 8 * (sub - 4);
        const uint32_t lo = (s2 >> sh) & 0xFFu;
        *sc = (lo & 0x0Fu) | ((((s0 >> sh) >> 6) & 0x3u) << 4);
        *mn = (lo >> 4) | ((((s1 >> sh) >> 6) & 0x3u) << 4);
    }
}

// q5_K: fp16 d, fp16 dmin, 12 scale bytes (as q4_K), 32 high-bit bytes at 16
// (bit 2g+s of byte l is bit 4 of value 64g+32s+l), 128 nibble bytes at 48
// (nibble s of byte 32g+l).  value = d*sc*q - dmin*m.
struct FmtQ5_K {
    static constexpr int QK = 256, BYTES = 176, NW = 8;
    __device__ static void fetch(const uint8_t *blk, int w, uint32_t (&r)[NW]) {
        const int g = w >> 6, l0 = w & 31;
        r[0] = ld_u32(blk);
        r[1] = ld_u32(blk + 4);
        r[2] = ld_u32(blk + 8);
        r[3] = ld_u32(blk + 12);
        r[4] = ld_u32(blk + 16 + l0);
        r[5] = ld_u32(blk + 20 + l0);
        r[6] = ld_u32(blk + 48 + 32 * g + l0);
        r[7] = ld_u32(blk + 52 + 32 * g + l0);
    }
    __device__ static void decode(const uint32_t (&r)[NW], int w, float (&v)[8]) {
        const int sub = w >> 5, g = w >> 6, s = (w >> 5) & 1;
        uint32_t sc, mn;
        k4_scale_min(r[1], r[2], r[3], sub, &sc, &mn);
        const float ds = half_bits_to_float(r[0] & 0xFFFFu) * (float)sc;
        const float dm = half_bits_to_float(r[0] >> 16) * (float)mn;
        const int hs = 2 * g + s;
        const uint32_t n0 = opaque(((r[6] >> (4 * s)) & 0x0F0F0F0Fu) | (((r[4] >> hs) & 0x01010101u) << 4));
        const uint32_t n1 = opaque(((r[7] >> (4 * s)) & 0x0F0F0F0Fu) | (((r[5] >> hs) & 0x01010101u) << 4));
#pragma unroll
        for (int e = 0; e < 4; ++e) {  // ds*q exact, one rounding with - dm
            v[e] = __builtin_fmaf(ds, ubyte(n0, e), -dm);
            v[4 + e] = __builtin_fmaf(ds, ubyte(n1, e), -dm);
        }
    }
};

// q6_K: 128 nibble bytes (value 128h+32c+l: nibble c/2 of byte
// 64h + 32(c%2) + l), 64 bytes of top bit pairs at 128 (bits 2c..2c+1 of
// byte 32h + l), 16 int8 scales at 192 (sub-blocks of 16), fp16 d at 208.
// value = d*scale*(q - 32).
struct FmtQ6_K {
    static constexpr int QK = 256, BYTES = 210, NW = 6;
    __device__ static void fetch(const uint8_t *blk, int w, uint32_t (&r)[NW]) {
        const int h = w >> 7, c = (w >> 5) & 3, l0 = w & 31;
        const int lo = 64 * h + 32 * (c & 1) + l0;
        r[0] = ld_u16(blk + 208);
        r[1] = ld_u32_a2(blk + lo);
        r[2] = ld_u32_a2(blk + lo + 4);
        r[3] = ld_u32_a2(blk + 128 + 32 * h + l0);
        r[4] = ld_u32_a2(blk + 132 + 32 * h + l0);
        r[5] = ld_u16(blk + 192 + 2 * (w >> 5));  // scale bytes w/16 (and its pair)
    }
    __device__ static void decode(const uint32_t (&r)[NW], int w, float (&v)[8]) {
        const int c = (w >> 5) & 3;
        const int sc = (int)(int8_t)((r[5] >> (8 * ((w >> 4) & 1))) & 0xFFu);
        const float ds = half_bits_to_float(r[0]) * (float)sc;  // exact: <= 19 bits
        const int ns = 4 * (c >> 1);
        const uint32_t u0 = opaque(((r[1] >> ns) & 0x0F0F0F0Fu) | (((r[3] >> (2 * c)) & 0x03030303u) << 4));
        const uint32_t u1 = opaque(((r[2] >> ns) & 0x0F0F0F0Fu) | (((r[4] >> (2 * c)) & 0x03030303u) << 4));
        const float off = -32.f * ds;  // exact
#pragma unroll
        for (int e = 0; e < 4; ++e) {  // ds*(u - 32) rounded once, as d*scale*q
            v[e] = __builtin_fmaf(ds, ubyte(u0, e), off);
            v[4 + e] = __builtin_fmaf(ds, ubyte(u1, e), off);
        }
    }
};

}  // namespace outprod
