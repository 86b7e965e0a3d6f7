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
 * f32 grad", q8_0 weights in the gate test -- but not their bytes; the
 * layouts below are the GGUF block formats as publicly documented):
 *   q8_0, 34 bytes / 32 values: bytes 0-1 fp16 d; bytes 2..33 int8 q[32].
 *   q4_K, 144 bytes / 256 values: bytes 0-1 fp16 d, 2-3 fp16 dmin,
 *     4..15 twelve bytes of packed 6-bit (scale, min) for 8 sub-blocks of 32,
 *     16..143 128 bytes of 4-bit q.  See q4k_subblock_params and
 *     decode_q4_K_row for the exact bit positions.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_F32 0
#define ORC_Q8_0 8
#define ORC_Q4_K 12

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

static int block_size(int a_type)
{
    return a_type == ORC_Q8_0 ? 32 : a_type == ORC_Q4_K ? 256 : 1;
}

/* Decode nrows rows of ne00 values each.  Row r starts at byte r*row_stride. */
int oracle_dequant_rows(const void *a, int a_type, int64_t ne00, int64_t nrows,
                        int64_t row_stride, float *out)
{
    if (!a || !out || ne00 < 0 || nrows < 0)
        return ORC_E_ARG;
    if (ne00 % block_size(a_type) != 0)
        return ORC_E_SHAPE;
    for (int64_t r = 0; r < nrows; ++r) {
        const uint8_t *row = (const uint8_t *)a + r * row_stride;
        float *o = out + r * ne00;
        int rc = ORC_OK;
        if (a_type == ORC_F32)
            memcpy(o, row, (size_t)ne00 * sizeof(float));
        else if (a_type == ORC_Q8_0)
            rc = decode_q8_0_row(row, ne00, o);
        else if (a_type == ORC_Q4_K)
            rc = decode_q4_K_row(row, ne00, o);
        else
            return ORC_E_ARG;
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
    if (a_type != ORC_F32 && a_type != ORC_Q8_0 && a_type != ORC_Q4_K)
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
