/*
 * oracle.c -- plain CPU oracle for ggml's OUT_PROD, in double precision.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library never
 * links, includes or calls it, and it shares no code with the GPU library:
 * this file has its own fp16 decoder, its own q8_0 / q4_K decoders and its
 * own slice mapping.
 *
 * What it computes (pages: "metal: OUT_PROD runs batched, broadcast and
 * narrow shapes on the GPU", review "VERIFIED BY READING": the op builds dst
 * as {a.ne0, b.ne0, b.ne2, b.ne3}, requires b.ne2 % a.ne2 == 0 and
 * b.ne3 % a.ne3 == 0, and maps slices with the CPU backend's rule
 * i02 = i2/dps2; and the body's "per-slice helper ... dps2 = ne2/ne02"):
 *
 *   dps2 = ne12/ne02, dps3 = ne13/ne03, i02 = i2/dps2, i03 = i3/dps3
 *   ref[i0,i1,i2,i3] = sum_{k=0}^{K-1} A(i0,k,i02,i03) * B(i1,k,i2,i3)
 *   den[i0,i1,i2,i3] = sum_{k=0}^{K-1} |A(i0,k,i02,i03)| * |B(i1,k,i2,i3)|
 *
 * Both sums are taken in double, k ascending.  A product of two floats is
 * exact in double (24+24 <= 53 significand bits), so the only roundings are
 * those of the double additions.
 *
 * Dequantized values are defined as float: the exact value of the block's
 * formula, rounded once to nearest float (a dequantized weight row is a
 * float row).  For q8_0 (value = d*q) the product is exact in float already;
 * for q4_K (value = d*sc*q - dmin*m) every term is exact and only the final
 * difference rounds.  The oracle forms the exact difference in double and
 * converts to float, which is that single round-to-nearest-even.
 *
 * Block layouts (the pages name the types -- a Q4_K_M model, "q4_K weight x
 * f32 grad", q8_0 weights in the gate test, and the MUL_MAT_ID_BACK page's
 * list of the frozen-weight types out_prod reads: f32, f16, bf16, q4_0,
 * q4_1, q5_0, q5_1, q8_0, q2_K..q6_K -- but not their bytes; the layouts
 * below are the GGUF block formats as publicly documented, multi-byte
 * fields little-endian):
 *   f16 / bf16, 2 bytes / 1 value: IEEE binary16 / the top half of a binary32.
 *   q4_0, 18 bytes / 32: fp16 d; 16 bytes of 4-bit q; value = d*(q-8).
 *   q4_1, 20 bytes / 32: fp16 d, fp16 m; 16 bytes of 4-bit q; value = d*q + m.
 *   q5_0, 22 bytes / 32: fp16 d; 32 high bits; 16 bytes of low nibbles;
 *     value = d*(q-16).
 *   q5_1, 24 bytes / 32: fp16 d, fp16 m; 32 high bits; 16 bytes of low
 *     nibbles; value = d*q + m.
 *   q8_0, 34 bytes / 32: fp16 d; bytes 2..33 int8 q[32]; value = d*q.
 *   q2_K, 84 bytes / 256: 16 bytes of (4-bit scale, 4-bit min) for 16
 *     sub-blocks of 16; 64 bytes of 2-bit q; fp16 d; fp16 dmin;
 *     value = d*scale*q - dmin*min.
 *   q3_K, 110 bytes / 256: 32 bytes of high bits; 64 bytes of 2-bit low
 *     parts; 12 bytes of 6-bit scales for 16 sub-blocks; fp16 d;
 *     value = d*(scale-32)*q with q in [-4, 3].
 *   q4_K, 144 bytes / 256: bytes 0-1 fp16 d, 2-3 fp16 dmin,
 *     4..15 twelve bytes of packed 6-bit (scale, min) for 8 sub-blocks of 32,
 *     16..143 128 bytes of 4-bit q; value = d*scale*q - dmin*min.
 *   q5_K, 176 bytes / 256: as q4_K plus 32 bytes of high bits before the
 *     nibbles; q has 5 bits.
 *   q6_K, 210 bytes / 256: 128 bytes of low nibbles; 64 bytes of 2-bit high
 *     parts; 16 int8 scales for sub-blocks of 16; fp16 d;
 *     value = d*scale*(q-32).
 * The decoders below state the exact bit positions.  Every value is the
 * exact block formula rounded once to float (for q3_K and the 32-value
 * types without an offset the formula is exact in float already).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_F32 0
#define ORC_F16 1
#define ORC_Q4_0 2
#define ORC_Q4_1 3
#define ORC_Q5_0 6
#define ORC_Q5_1 7
#define ORC_Q8_0 8
#define ORC_Q2_K 10
#define ORC_Q3_K 11
#define ORC_Q4_K 12
#define ORC_Q5_K 13
#define ORC_Q6_K 14
#define ORC_BF16 30

#define ORC_OK 0
#define ORC_E_ARG (-1)
#define ORC_E_SHAPE (-2)
#define ORC_E_FP16 (-3)
#define ORC_E_NOMEM (-4)

/* IEEE binary16 bits -> double, exactly.  Normal numbers are
 * (1024 + f) * 2^(e-25); subnormals are f * 2^-24.  Inf and NaN are refused
 * (returns -1): a weight scale is a finite number. */
static int half_to_double(uint16_t h, double *out)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 31)
        return -1;
    if (e == 0)
        v = ldexp((double)f, -24);
    else
        v = ldexp((double)(1024 + f), e - 25);
    *out = sign ? -v : v;
    return 0;
}

static uint16_t load_u16le(const uint8_t *p)
{
    return (uint16_t)(p[0] | ((uint16_t)p[1] << 8));
}

/* q8_0: x[j] = d * q[j] for the 32 values of a block. */
static int decode_q8_0_row(const uint8_t *row, int64_t n, float *out)
{
    for (int64_t blk = 0; blk < n / 32; ++blk) {
        const uint8_t *p = row + 34 * blk;
        double d;
        if (half_to_double(load_u16le(p), &d))
            return ORC_E_FP16;
        for (int j = 0; j < 32; ++j) {
            int q = (int)(int8_t)p[2 + j];
            out[32 * blk + j] = (float)(d * (double)q);
        }
    }
    return ORC_OK;
}

/* q4_K packing of the eight 6-bit scales sc[j] and mins m[j] in 12 bytes s[]:
 *   s[0..3]  : bits 0-5 = sc[0..3], bits 6-7 = bits 4-5 of sc[4..7]
 *   s[4..7]  : bits 0-5 =  m[0..3], bits 6-7 = bits 4-5 of  m[4..7]
 *   s[8..11] : bits 0-3 = bits 0-3 of sc[4..7], bits 4-7 = bits 0-3 of m[4..7]
 */
static void q4k_subblock_params(const uint8_t *s, int j, int *sc, int *m)
{
    if (j < 4) {
        *sc = s[j] & 0x3F;
        *m = s[j + 4] & 0x3F;
    } else {
        int lo_sc = s[j + 4] & 0x0F;   /* s[8 + (j-4)] */
        int lo_m = s[j + 4] >> 4;
        int hi_sc = s[j - 4] >> 6;     /* top bits of s[0 + (j-4)] */
        int hi_m = s[j] >> 6;          /* top bits of s[4 + (j-4)] */
        *sc = lo_sc | (hi_sc << 4);
        *m = lo_m | (hi_m << 4);
    }
}

/* q4_K: 256 values = 4 groups of 64.  In group g, the 32 bytes
 * qs[32g .. 32g+31] hold value i of sub-block 2g in their low nibble and value
 * i of sub-block 2g+1 in their high nibble.  Value = d*sc*q - dmin*m. */
static int decode_q4_K_row(const uint8_t *row, int64_t n, float *out)
{
    for (int64_t blk = 0; blk < n / 256; ++blk) {
        const uint8_t *p = row + 144 * blk;
        const uint8_t *scales = p + 4;
        const uint8_t *qs = p + 16;
        double d, dmin;
        if (half_to_double(load_u16le(p), &d) || half_to_double(load_u16le(p + 2), &dmin))
            return ORC_E_FP16;
        for (int j = 0; j < 8; ++j) {
            int sc, m;
            q4k_subblock_params(scales, j, &sc, &m);
            for (int i = 0; i < 32; ++i) {
                uint8_t byte = qs[32 * (j / 2) + i];
                int q = (j % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
                double exact = d * (double)sc * (double)q - dmin * (double)m;
                out[256 * blk + 32 * j + i] = (float)exact;
            }
        }
    }
    return ORC_OK;
}

/* bfloat16 bits -> double: the 16 bits are the top half of a binary32, so
 * the value is that float's.  Inf and NaN are refused (returns -1). */
static int bf16_to_double(uint16_t h, double *out)
{
    if (((h >> 7) & 0xFF) == 0xFF)
        return -1;
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    *out = (double)f;
    return 0;
}

/* f16 and bf16 rows: one 2-byte value per element. */
static int decode_f16_row(const uint8_t *row, int64_t n, int bf16, float *out)
{
    for (int64_t i = 0; i < n; ++i) {
        double v;
        uint16_t h = load_u16le(row + 2 * i);
        if (bf16 ? bf16_to_double(h, &v) : half_to_double(h, &v))
            return ORC_E_FP16;
        out[i] = (float)v;
    }
    return ORC_OK;
}

/* The 32-value types.  Value j of a block (j < 16: the low nibble of code
 * byte j; j >= 16: the high nibble of code byte j-16); q5_0 / q5_1 add bit j
 * of the 32-bit high-bit word as bit 4 of q.  Offsets of the fields:
 *   q4_0: d 0, codes 2        q4_1: d 0, m 2, codes 4
 *   q5_0: d 0, high 2, codes 6  q5_1: d 0, m 2, high 4, codes 8 */
static int decode_small_row(const uint8_t *row, int64_t n, int type, float *out)
{
    const int bytes = type == ORC_Q4_0 ? 18 : type == ORC_Q4_1 ? 20 : type == ORC_Q5_0 ? 22 : 24;
    const int has_m = type == ORC_Q4_1 || type == ORC_Q5_1;
    const int five = type == ORC_Q5_0 || type == ORC_Q5_1;
    const int off_high = has_m ? 4 : 2;
    const int off_codes = (has_m ? 4 : 2) + (five ? 4 : 0);
    for (int64_t blk = 0; blk < n / 32; ++blk) {
        const uint8_t *p = row + (int64_t)bytes * blk;
        double d, m = 0.0;
        if (half_to_double(load_u16le(p), &d))
            return ORC_E_FP16;
        if (has_m && half_to_double(load_u16le(p + 2), &m))
            return ORC_E_FP16;
        uint32_t high = 0;
        if (five)
            high = (uint32_t)p[off_high] | ((uint32_t)p[off_high + 1] << 8) |
                   ((uint32_t)p[off_high + 2] << 16) | ((uint32_t)p[off_high + 3] << 24);
        for (int j = 0; j < 32; ++j) {
            const uint8_t byte = p[off_codes + (j % 16)];
            int q = j < 16 ? (byte & 0x0F) : (byte >> 4);
            if (five)
                q |= (int)((high >> j) & 1u) << 4;
            double exact;
            if (has_m)
                exact = d * (double)q + m;
            else
                exact = d * (double)(q - (five ? 16 : 8));
            out[32 * blk + j] = (float)exact;
        }
    }
    return ORC_OK;
}

/* q2_K (84 bytes): scales[16] at 0, codes[64] at 16, fp16 d at 80, fp16
 * dmin at 82.  Value v = 128h + 32j + t (h < 2, j < 4, t < 32): q = bits
 * 2j..2j+1 of code byte 32h + t; sub-block v/16 has scale = low nibble and
 * min = high nibble of scales[v/16].  Value = d*scale*q - dmin*min. */
static int decode_q2_K_row(const uint8_t *row, int64_t n, float *out)
{
    for (int64_t blk = 0; blk < n / 256; ++blk) {
        const uint8_t *p = row + 84 * blk;
        double d, dmin;
        if (half_to_double(load_u16le(p + 80), &d) || half_to_double(load_u16le(p + 82), &dmin))
            return ORC_E_FP16;
        for (int v = 0; v < 256; ++v) {
            const int h = v / 128, j = (v % 128) / 32, t = v % 32;
            const int q = (p[16 + 32 * h + t] >> (2 * j)) & 3;
            const int sm = p[v / 16];
            double exact = d * (double)(sm & 0x0F) * (double)q - dmin * (double)(sm >> 4);
            out[256 * blk + v] = (float)exact;
        }
    }
    return ORC_OK;
}

/* q3_K (110 bytes): high-bit mask[32] at 0, codes[64] at 32, scales[12] at
 * 96, fp16 d at 108.  Value v = 128h + 32j + t: low two bits = bits 2j..2j+1
 * of code byte 32h + t; high bit = bit 4h + j of mask byte t; q = low - 4
 * when the high bit is clear, else low.  Scale i = v/16 (6 bits, stored
 * biased by 32): low four bits = low nibble of byte i (i < 8) or high nibble
 * of byte i - 8 (i >= 8); top two bits = bits 2*(i/4)..+1 of byte 8 + i%4 of
 * the scale field.  Value = d*(scale - 32)*q. */
static int decode_q3_K_row(const uint8_t *row, int64_t n, float *out)
{
    for (int64_t blk = 0; blk < n / 256; ++blk) {
        const uint8_t *p = row + 110 * blk;
        const uint8_t *mask = p, *codes = p + 32, *sc = p + 96;
        double d;
        if (half_to_double(load_u16le(p + 108), &d))
            return ORC_E_FP16;
        for (int v = 0; v < 256; ++v) {
            const int h = v / 128, j = (v % 128) / 32, t = v % 32;
            const int low = (codes[32 * h + t] >> (2 * j)) & 3;
            const int hb = (mask[t] >> (4 * h + j)) & 1;
            const int q = hb ? low : low - 4;
            const int i = v / 16;
            const int lo4 = i < 8 ? (sc[i] & 0x0F) : (sc[i - 8] >> 4);
            const int hi2 = (sc[8 + i % 4] >> (2 * (i / 4))) & 3;
            const int scale = (lo4 | (hi2 << 4)) - 32;
            out[256 * blk + v] = (float)(d * (double)scale * (double)q);
        }
    }
    return ORC_OK;
}

/* q5_K (176 bytes): fp16 d at 0, fp16 dmin at 2, scales[12] at 4 (packed as
 * in q4_K), high bits[32] at 16, nibbles[128] at 48.  Value v = 64g + 32s + l:
 * the low four bits are nibble s (0: low, 1: high) of byte 32g + l; bit 4 is
 * bit 2g + s of high-bit byte l; sub-block v/32.  Value = d*sc*q - dmin*m. */
static int decode_q5_K_row(const uint8_t *row, int64_t n, float *out)
{
    for (int64_t blk = 0; blk < n / 256; ++blk) {
        const uint8_t *p = row + 176 * blk;
        const uint8_t *high = p + 16, *qs = p + 48;
        double d, dmin;
        if (half_to_double(load_u16le(p), &d) || half_to_double(load_u16le(p + 2), &dmin))
            return ORC_E_FP16;
        for (int v = 0; v < 256; ++v) {
            const int g = v / 64, s = (v % 64) / 32, l = v % 32;
            const uint8_t byte = qs[32 * g + l];
            int q = s ? (byte >> 4) : (byte & 0x0F);
            q |= ((high[l] >> (2 * g + s)) & 1) << 4;
            int sc, m;
            q4k_subblock_params(p + 4, v / 32, &sc, &m);
            out[256 * blk + v] = (float)(d * (double)sc * (double)q - dmin * (double)m);
        }
    }
    return ORC_OK;
}

/* q6_K (210 bytes): low nibbles[128] at 0, high parts[64] at 128, int8
 * scales[16] at 192, fp16 d at 208.  Value v = 128h + 32c + l (c < 4): low
 * four bits = nibble c/2 (0: low, 1: high) of byte 64h + 32(c%2) + l; top two
 * bits = bits 2c..2c+1 of high byte 32h + l; q = that 6-bit number - 32;
 * scale = scales[v/16].  Value = d*scale*q. */
static int decode_q6_K_row(const uint8_t *row, int64_t n, float *out)
{
    for (int64_t blk = 0; blk < n / 256; ++blk) {
        const uint8_t *p = row + 210 * blk;
        const uint8_t *ql = p, *qh = p + 128;
        const int8_t *sc = (const int8_t *)(p + 192);
        double d;
        if (half_to_double(load_u16le(p + 208), &d))
            return ORC_E_FP16;
        for (int v = 0; v < 256; ++v) {
            const int h = v / 128, c = (v % 128) / 32, l = v % 32;
            const uint8_t lb = ql[64 * h + 32 * (c % 2) + l];
            const int low = c < 2 ? (lb & 0x0F) : (lb >> 4);
            const int top = (qh[32 * h + l] >> (2 * c)) & 3;
            const int q = (low | (top << 4)) - 32;
            out[256 * blk + v] = (float)(d * (double)sc[v / 16] * (double)q);
        }
    }
    return ORC_OK;
}

static int block_size(int a_type)
{
    switch (a_type) {
    case ORC_Q4_0: case ORC_Q4_1: case ORC_Q5_0: case ORC_Q5_1: case ORC_Q8_0: return 32;
    case ORC_Q2_K: case ORC_Q3_K: case ORC_Q4_K: case ORC_Q5_K: case ORC_Q6_K: return 256;
    default: return 1;
    }
}

static int known_type(int t)
{
    switch (t) {
    case ORC_F32: case ORC_F16: case ORC_BF16: case ORC_Q4_0: case ORC_Q4_1: case ORC_Q5_0:
    case ORC_Q5_1: case ORC_Q8_0: case ORC_Q2_K: case ORC_Q3_K: case ORC_Q4_K: case ORC_Q5_K:
    case ORC_Q6_K: return 1;
    default: return 0;
    }
}

/* Decode nrows rows of ne00 values each.  Row r starts at byte r*row_stride. */
int oracle_dequant_rows(const void *a, int a_type, int64_t ne00, int64_t nrows,
                        int64_t row_stride, float *out)
{
    if (!a || !out || ne00 < 0 || nrows < 0 || !known_type(a_type))
        return ORC_E_ARG;
    if (ne00 % block_size(a_type) != 0)
        return ORC_E_SHAPE;
    for (int64_t r = 0; r < nrows; ++r) {
        const uint8_t *row = (const uint8_t *)a + r * row_stride;
        float *o = out + r * ne00;
        int rc = ORC_OK;
        switch (a_type) {
        case ORC_F32: memcpy(o, row, (size_t)ne00 * sizeof(float)); break;
        case ORC_F16: rc = decode_f16_row(row, ne00, 0, o); break;
        case ORC_BF16: rc = decode_f16_row(row, ne00, 1, o); break;
        case ORC_Q4_0: case ORC_Q4_1: case ORC_Q5_0: case ORC_Q5_1:
            rc = decode_small_row(row, ne00, a_type, o);
            break;
        case ORC_Q8_0: rc = decode_q8_0_row(row, ne00, o); break;
        case ORC_Q2_K: rc = decode_q2_K_row(row, ne00, o); break;
        case ORC_Q3_K: rc = decode_q3_K_row(row, ne00, o); break;
        case ORC_Q4_K: rc = decode_q4_K_row(row, ne00, o); break;
        case ORC_Q5_K: rc = decode_q5_K_row(row, ne00, o); break;
        case ORC_Q6_K: rc = decode_q6_K_row(row, ne00, o); break;
        default: return ORC_E_ARG;
        }
        if (rc)
            return rc;
    }
    return ORC_OK;
}

/*
 * ne[12], nb[12]: a.ne[0..3], b.ne[0..3], dst.ne[0..3] and the byte strides
 * in the same order (ggml's convention; for a quantized a, nb[0] is the block
 * size in bytes and nb[1] the byte stride between the rows k).
 *
 * cols: ncols triples (i1, i2, i3) naming the dst columns dst[:, i1, i2, i3]
 * to compute, or NULL for every column in dst order (i1 fastest, then i2,
 * then i3; ncols is then ignored).  ref and den receive ne00 doubles per
 * column, column after column.
 */
int oracle_out_prod(const void *a, int a_type, const float *b,
                    const int64_t ne[12], const int64_t nb[12],
                    const int64_t *cols, int64_t ncols, double *ref, double *den)
{
    if (!ne || !nb || !ref || !den)
        return ORC_E_ARG;
    const int64_t ne00 = ne[0], K = ne[1], ne02 = ne[2], ne03 = ne[3];
    const int64_t ne10 = ne[4], ne11 = ne[5], ne12 = ne[6], ne13 = ne[7];
    for (int i = 0; i < 12; ++i)
        if (ne[i] < 0)
            return ORC_E_SHAPE;
    if (ne11 != K || ne[8] != ne00 || ne[9] != ne10 || ne[10] != ne12 || ne[11] != ne13)
        return ORC_E_SHAPE;
    if (ne02 < 1 || ne03 < 1 || ne12 % ne02 != 0 || ne13 % ne03 != 0)
        return ORC_E_SHAPE;
    if (!known_type(a_type))
        return ORC_E_ARG;
    if (ne00 % block_size(a_type) != 0)
        return ORC_E_SHAPE;
    if (!cols)
        ncols = ne10 * ne12 * ne13;
    if (ncols == 0 || ne00 == 0)
        return ORC_OK;
    if (K > 0 && (!a || !b))
        return ORC_E_ARG;

    const int64_t dps2 = ne12 / ne02, dps3 = ne13 / ne03;

    /* Decode every a slice into float rows [i03][i02][k][i0]. */
    const int64_t slice_vals = K * ne00;
    float *A = NULL;
    if (slice_vals > 0) {
        A = (float *)malloc((size_t)(slice_vals * ne02 * ne03) * sizeof(float));
        if (!A)
            return ORC_E_NOMEM;
        int bad = 0;
#pragma omp parallel for collapse(2) schedule(static) reduction(| : bad)
        for (int64_t i03 = 0; i03 < ne03; ++i03)
            for (int64_t i02 = 0; i02 < ne02; ++i02) {
                const uint8_t *base = (const uint8_t *)a + i02 * nb[2] + i03 * nb[3];
                float *out = A + (i03 * ne02 + i02) * slice_vals;
                if (oracle_dequant_rows(base, a_type, ne00, K, nb[1], out))
                    bad |= 1;
            }
        if (bad) {
            free(A);
            return ORC_E_FP16;
        }
    }

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t c = 0; c < ncols; ++c) {
        int64_t i1, i2, i3;
        if (cols) {
            i1 = cols[3 * c + 0];
            i2 = cols[3 * c + 1];
            i3 = cols[3 * c + 2];
        } else {
            i1 = c % ne10;
            i2 = (c / ne10) % ne12;
            i3 = c / (ne10 * ne12);
        }
        double *r = ref + c * ne00;
        double *dn = den + c * ne00;
        for (int64_t i0 = 0; i0 < ne00; ++i0) {
            r[i0] = 0.0;
            dn[i0] = 0.0;
        }
        if (i1 < 0 || i1 >= ne10 || i2 < 0 || i2 >= ne12 || i3 < 0 || i3 >= ne13)
            continue; /* out-of-range request: left at zero */
        const int64_t i02 = i2 / dps2, i03 = i3 / dps3;
        const float *As = A ? A + (i03 * ne02 + i02) * slice_vals : NULL;
        const uint8_t *bcol = (const uint8_t *)b + i1 * nb[4] + i2 * nb[6] + i3 * nb[7];
        for (int64_t k = 0; k < K; ++k) {
            const double bk = (double)*(const float *)(bcol + k * nb[5]);
            const double abk = fabs(bk);
            const float *arow = As + k * ne00;
            for (int64_t i0 = 0; i0 < ne00; ++i0) {
                const double av = (double)arow[i0];
                r[i0] += av * bk;
                dn[i0] += fabs(av) * abk;
            }
        }
    }
    free(A);
    return ORC_OK;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/*
 * MUL_MAT_ID_BACK: the input gradient of MUL_MAT_ID through frozen experts
 * (pages: the MUL_MAT_ID_BACK Metal-kernel page -- one writer per element of
 * a routed slot's row, the expert's rows walked, experts dequantized from the
 * same types as out_prod's a; its proof is the gradient check of MUL_MAT_ID).
 *
 * Reading (the op's CPU definition is not on the pages): MUL_MAT_ID's slot
 * (i, t) multiplies its input row by expert e = ids[i, t], so its input
 * gradient is, for every slot (i < n_used, t < n_tokens) and c < ne00,
 *
 *   ref[t][i][c] = sum_{r<K} A_e(c, r) * g(r, i, t)
 *   den[t][i][c] = sum_{r<K} |A_e(c, r)| * |g(r, i, t)|
 *
 * with A_e(c, r) the dequantized value c of row r of expert e, summed in
 * double over r ascending.  Tensors (ggml order, byte strides):
 *   ne[0..3]  as  = {ne00, K, n_expert, 1}   nb[0] = element or block bytes
 *   ne[4..7]  g   = {K, n_used, n_tokens, 1} nb[4] = 4 (r contiguous)
 *   ne[8..11] ids = {n_used, n_tokens, 1, 1} int32, nb[8] = 4
 *   ne[12..15] dst = {ne00, n_used, n_tokens, 1} (shape check only)
 * slots: nslots slot numbers s = i + n_used*t to compute (ref/den receive
 * ne00 doubles per listed slot), or NULL for every slot in s order.  An id
 * outside [0, n_expert) is refused (ORC_E_ARG).
 */
int oracle_mul_mat_id_back(const void *as, int as_type, const float *g, const int32_t *ids,
                           const int64_t ne[16], const int64_t nb[16], const int64_t *slots,
                           int64_t nslots, double *ref, double *den)
{
    if (!ne || !nb || !ref || !den || !known_type(as_type))
        return ORC_E_ARG;
    for (int i = 0; i < 16; ++i)
        if (ne[i] < 0)
            return ORC_E_SHAPE;
    const int64_t ne00 = ne[0], K = ne[1], n_expert = ne[2];
    const int64_t n_used = ne[5], n_tokens = ne[6];
    if (ne[3] != 1 || ne[4] != K || ne[7] != 1 || ne[8] != n_used || ne[9] != n_tokens ||
        ne[10] != 1 || ne[11] != 1 || ne[12] != ne00 || ne[13] != n_used || ne[14] != n_tokens ||
        ne[15] != 1)
        return ORC_E_SHAPE;
    if (ne00 % block_size(as_type) != 0 || nb[4] != 4 || nb[8] != 4)
        return ORC_E_SHAPE;
    const int64_t total = n_used * n_tokens;
    if (!slots)
        nslots = total;
    if (nslots == 0 || ne00 == 0)
        return ORC_OK;
    if (!ids || (K > 0 && (!as || !g)))
        return ORC_E_ARG;
    for (int64_t q = 0; q < nslots; ++q) {
        const int64_t s = slots ? slots[q] : q;
        if (s < 0 || s >= total)
            return ORC_E_ARG;
        const int64_t i = s % n_used, t = s / n_used;
        const int32_t e = *(const int32_t *)((const uint8_t *)ids + i * 4 + t * nb[9]);
        if (e < 0 || e >= n_expert)
            return ORC_E_ARG;
    }

    /* one expert at a time: decode its K rows, then every listed slot routed to it */
    float *A = NULL;
    if (K > 0) {
        A = (float *)malloc((size_t)(K * ne00) * sizeof(float));
        if (!A)
            return ORC_E_NOMEM;
    }
    int rc = ORC_OK;
    for (int64_t e = 0; e < n_expert && rc == ORC_OK; ++e) {
        int used = 0;
        for (int64_t q = 0; q < nslots && !used; ++q) {
            const int64_t s = slots ? slots[q] : q;
            used = *(const int32_t *)((const uint8_t *)ids + (s % n_used) * 4 + (s / n_used) * nb[9]) == e;
        }
        if (!used)
            continue;
        if (K > 0 && oracle_dequant_rows((const uint8_t *)as + e * nb[2], as_type, ne00, K, nb[1], A)) {
            rc = ORC_E_FP16;
            break;
        }
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t q = 0; q < nslots; ++q) {
            const int64_t s = slots ? slots[q] : q;
            const int64_t i = s % n_used, t = s / n_used;
            if (*(const int32_t *)((const uint8_t *)ids + i * 4 + t * nb[9]) != e)
                continue;
            double *r = ref + q * ne00;
            double *dn = den + q * ne00;
            for (int64_t c = 0; c < ne00; ++c) {
                r[c] = 0.0;
                dn[c] = 0.0;
            }
            const uint8_t *gcol = (const uint8_t *)g + i * nb[5] + t * nb[6];
            for (int64_t k = 0; k < K; ++k) {
                const double gk = (double)*(const float *)(gcol + 4 * k);
                const double agk = fabs(gk);
                const float *Ak = A + k * ne00;
                for (int64_t c = 0; c < ne00; ++c) {
                    r[c] += (double)Ak[c] * gk;
                    dn[c] += fabs((double)Ak[c]) * agk;
                }
            }
        }
    }
    /* K == 0: every listed slot's row is an empty sum */
    if (K == 0)
        for (int64_t q = 0; q < nslots * ne00; ++q)
            ref[q] = den[q] = 0.0;
    free(A);
    return rc;
}
