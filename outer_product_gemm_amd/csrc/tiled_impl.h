// tiled_impl.h -- the tiled OUT_PROD kernel template, its operand loaders
// and its configuration menu.  Included by the per-type instantiation files
// (tiled_*.hip) and by the planner (kernel_tiled.hip).
//
// OUT_PROD for wide problems: frozen quantized weight x f32
// gradient products and other shapes with many flops per byte (pages: "metal:
// OUT_PROD runs batched, broadcast and narrow shapes on the GPU" -- every
// (i2, i3) slice in one launch instead of one encode per slice; "metal:
// OUT_PROD multiplies in float staging" -- fp32 staging of both operands; and
// the MUL_MAT_ID_BACK page's note that quantized rows are dequantized in
// registers rather than copied to a scratch buffer).
//
// In BLAS terms each slice is dst(N x M, row-major) = B^T A with A = a's
// [K][M] rows and B = b's [K][N] rows: both operands are K-major, so a K-tile
// of either is BK contiguous row segments.  A workgroup owns a BM x BN dst
// tile (BM along i0, BN along i1) of one slice and walks K in BK-row stages:
//   global -> registers (a: f32 copy, f16/bf16 widening or a block decode
//   to fp32;
//   b: f32) -> LDS [k][i0] / [k][i1] (fp32, two buffers) ->
//   v_mfma_f32_{32x32x2,16x16x4}_f32 with fp32 accumulators.
// Pipeline: the registers hold stage t+1 while stage t is multiplied; halfway
// through stage t's MFMAs they are decoded into the other LDS buffer and the
// loads of stage t+2 are issued, so a global load has a whole stage of matrix
// work to arrive.  One barrier per stage.
// b may also have its K dim contiguous (the transposed gradient view of the
// matmul backward); that loader transposes into the same LDS tile.
// MFMA operand roles: A operand (rows) = b values -> dst rows i1;
// B operand (columns) = a values -> dst columns i0, so the lanes of one
// accumulator row write consecutive floats of a dst row.
#pragma once

#include <type_traits>

#include "block_formats.h"
#include "kernel_common.h"
#include "outprod.h"

namespace outprod {
namespace tiled {

// ---------------------------------------------------------------- loaders
// Each loader moves a BK x BW tile (BW columns of BK consecutive K rows) of
// one operand: load() issues the global reads of a stage into registers,
// store() converts them to fp32 and writes the LDS tile [k][column].
// Work is split into groups (4 floats, or 8 quantized values); thread tid
// takes groups tid, tid+T, ...; the last round is guarded when T does not
// divide the group count.

template <int BW, int BK, int T>
struct F32Loader {
    static constexpr int kGroups = BK * BW / 4;
    static constexpr int kPer = (kGroups + T - 1) / T;
    static_assert(BW % 4 == 0, "tile width must be a multiple of 4");
    const uint8_t *base;
    int64_t ld;
    int w0, W, K, tid;
    bool vec;
    floatx4 r[kPer];

    __device__ void init(const uint8_t *slice, int64_t row_stride, int width, int k_len,
                         int col0, bool vec_ok, int t) {
        base = slice;
        ld = row_stride;
        W = width;
        K = k_len;
        w0 = col0;
        vec = vec_ok;
        tid = t;
    }
    __device__ void load(int k0) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int g = tid + T * j;
            const int row = g / (BW / 4), c = w0 + 4 * (g % (BW / 4));
            const int k = k0 + row;
            floatx4 v = {0.f, 0.f, 0.f, 0.f};
            if ((kGroups % T == 0 || g < kGroups) && k < K) {
                const uint8_t *ptr = base + (int64_t)k * ld + (int64_t)c * 4;
                if (vec && c + 3 < W) {
                    v = *(const floatx4 *)ptr;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (c + e < W) v[e] = ldf(ptr + 4 * e);
                }
            }
            r[j] = v;
        }
    }
    template <int LD>
    __device__ void store(float (*lds)[LD]) const {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int g = tid + T * j;
            if (kGroups % T == 0 || g < kGroups) {
                const int row = g / (BW / 4), c = 4 * (g % (BW / 4));
                *(floatx4 *)&lds[row][c] = r[j];
            }
        }
    }
};

// f32 b whose K dim is contiguous (a transposed view; column stride `ld`):
// groups of 4 consecutive k of one column, written transposed into the same
// [k][column] LDS tile.
template <int BW, int BK, int T>
struct F32LoaderKT {
    static constexpr int kGroups = BK / 4 * BW;
    static constexpr int kPer = (kGroups + T - 1) / T;
    static_assert(BK % 4 == 0, "stage rows must be a multiple of 4");
    const uint8_t *base;
    int64_t ld;
    int w0, W, K, tid;
    bool vec;
    floatx4 r[kPer];

    __device__ void init(const uint8_t *slice, int64_t col_stride, int width, int k_len,
                         int col0, bool vec_ok, int t) {
        base = slice;
        ld = col_stride;
        W = width;
        K = k_len;
        w0 = col0;
        vec = vec_ok;
        tid = t;
    }
    __device__ void load(int k0) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int g = tid + T * j;
            const int n = g % BW, kq = g / BW;
            const int c = w0 + n, k = k0 + 4 * kq;
            floatx4 v = {0.f, 0.f, 0.f, 0.f};
            if ((kGroups % T == 0 || g < kGroups) && c < W) {
                const uint8_t *ptr = base + (int64_t)c * ld + (int64_t)k * 4;
                if (vec && k + 3 < K) {
                    v = *(const floatx4 *)ptr;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (k + e < K) v[e] = ldf(ptr + 4 * e);
                }
            }
            r[j] = v;
        }
    }
    template <int LD>
    __device__ void store(float (*lds)[LD]) const {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int g = tid + T * j;
            if (kGroups % T == 0 || g < kGroups) {
                const int n = g % BW, kq = g / BW;
#pragma unroll
                for (int e = 0; e < 4; ++e) lds[4 * kq + e][n] = r[j][e];
            }
        }
    }
};

// q8_0 a: groups of 8 consecutive values of one 32-value block.  34-byte
// blocks are only 2-byte aligned, so the codes come in as 16-bit loads.
template <int BM, int BK, int T>
struct Q8Loader {
    static constexpr int kGroups = BK * BM / 8;
    static constexpr int kPer = (kGroups + T - 1) / T;
    static_assert(BM % 8 == 0, "tile width must be a multiple of 8");
    const uint8_t *base;
    int64_t ld;
    int m0, M, K, tid;
    uint32_t d[kPer];
    uint32_t q[kPer][4];

    __device__ void init(const uint8_t *slice, int64_t row_stride, int width, int k_len,
                         int col0, bool, int t) {
        base = slice;
        ld = row_stride;
        M = width;
        K = k_len;
        m0 = col0;
        tid = t;
    }
    __device__ void load(int k0) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int g = tid + T * j;
            const int row = g / (BM / 8), m = m0 + 8 * (g % (BM / 8));
            const int k = k0 + row;
            d[j] = 0;
            q[j][0] = q[j][1] = q[j][2] = q[j][3] = 0;
            if ((kGroups % T == 0 || g < kGroups) && k < K && m < M) {
                const uint8_t *blk = base + (int64_t)k * ld + (int64_t)(m >> 5) * 34;
                const uint16_t *qs = (const uint16_t *)(blk + 2 + (m & 31));
                d[j] = *(const uint16_t *)blk;
#pragma unroll
                for (int e = 0; e < 4; ++e) q[j][e] = qs[e];
            }
        }
    }
    template <int LD>
    __device__ void store(float (*lds)[LD]) const {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int g = tid + T * j;
            if (!(kGroups % T == 0 || g < kGroups)) continue;
            const int row = g / (BM / 8), c = 8 * (g % (BM / 8));
            const float dd = half_bits_to_float(d[j]);
            float v[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // value = d * q, exact in fp32 (11 + 7 significant bits)
                v[2 * e] = dd * (float)(int8_t)(q[j][e] & 0xFFu);
                v[2 * e + 1] = dd * (float)(int8_t)(q[j][e] >> 8);
            }
            *(floatx4 *)&lds[row][c] = floatx4{v[0], v[1], v[2], v[3]};
            *(floatx4 *)&lds[row][c + 4] = floatx4{v[4], v[5], v[6], v[7]};
        }
    }
};

// q4_K a: groups of 8 consecutive values of one 32-value sub-block.
template <int BM, int BK, int T>
struct Q4KLoader {
    static constexpr int kGroups = BK * BM / 8;
    static constexpr int kPer = (kGroups + T - 1) / T;
    static_assert(BM % 8 == 0, "tile width must be a multiple of 8");
    const uint8_t *base;
    int64_t ld;
    int m0, M, K, tid;
    uint32_t dd[kPer], s0[kPer], s1[kPer], s2[kPer], q0[kPer], q1[kPer];

    __device__ void init(const uint8_t *slice, int64_t row_stride, int width, int k_len,
                         int col0, bool, int t) {
        base = slice;
        ld = row_stride;
        M = width;
        K = k_len;
        m0 = col0;
        tid = t;
    }
    __device__ void load(int k0) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int g = tid + T * j;
            const int row = g / (BM / 8), m = m0 + 8 * (g % (BM / 8));
            const int k = k0 + row;
            dd[j] = s0[j] = s1[j] = s2[j] = q0[j] = q1[j] = 0;
            if ((kGroups % T == 0 || g < kGroups) && k < K && m < M) {
                const uint8_t *blk = base + (int64_t)k * ld + (int64_t)(m >> 8) * 144;
                const int w = m & 255, sub = w >> 5, pos = w & 31;
                const uint32_t *hdr = (const uint32_t *)blk;
                const uint32_t *qs = (const uint32_t *)(blk + 16 + 32 * (sub >> 1) + pos);
                dd[j] = hdr[0];
                s0[j] = hdr[1];
                s1[j] = hdr[2];
                s2[j] = hdr[3];
                q0[j] = qs[0];
                q1[j] = qs[1];
            }
        }
    }
    template <int LD>
    __device__ void store(float (*lds)[LD]) const {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int g = tid + T * j;
            if (!(kGroups % T == 0 || g < kGroups)) continue;
            const int row = g / (BM / 8), c = 8 * (g % (BM / 8));
            const int sub = ((m0 + c) & 255) >> 5;
            // 6-bit scale and min of sub-block `sub` from the 12 packed bytes
            // (bytes 0-3 in s0, 4-7 in s1, 8-11 in s2): for sub < 4 the low 6
            // bits of bytes sub and 4+sub; otherwise the nibbles of byte
            // 8+(sub-4) below the top two bits of bytes sub-4 and sub.
            uint32_t sc, mn;
            if (sub < 4) {
                sc = (s0[j] >> (8 * sub)) & 0x3Fu;
                mn = (s1[j] >> (8 * sub)) & 0x3Fu;
            } else {
                const int sh = 8 * (sub - 4);
                const uint32_t lo = (s2[j] >> sh) & 0xFFu;
                sc = (lo & 0x0Fu) | ((((s0[j] >> sh) >> 6) & 0x3u) << 4);
                mn = (lo >> 4) | ((((s1[j] >> sh) >> 6) & 0x3u) << 4);
            }
            const float d = half_bits_to_float(dd[j] & 0xFFFFu);
            const float dmin = half_bits_to_float(dd[j] >> 16);
            const float ds = d * (float)sc;    // exact: <= 17 significant bits
            const float dm = dmin * (float)mn; // exact
            const int shift = (sub & 1) ? 4 : 0;
            float v[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // value = d*sc*q - dmin*m: the product is exact, one rounding
                v[e] = ds * (float)((q0[j] >> (8 * e + shift)) & 0xFu) - dm;
                v[4 + e] = ds * (float)((q1[j] >> (8 * e + shift)) & 0xFu) - dm;
            }
            *(floatx4 *)&lds[row][c] = floatx4{v[0], v[1], v[2], v[3]};
            *(floatx4 *)&lds[row][c + 4] = floatx4{v[4], v[5], v[6], v[7]};
        }
    }
};


// f16 / bf16 a: groups of 8 consecutive values of one row (any width; the
// group at the end of a row is guarded per element).  vec: rows 16-byte
// aligned, so a whole group is one 16-byte load.
template <bool BF, int BM, int BK, int T>
struct HalfLoader {
    static constexpr int kGroups = BK * BM / 8;
    static constexpr int kPer = (kGroups + T - 1) / T;
    static_assert(BM % 8 == 0, "tile width must be a multiple of 8");
    const uint8_t *base;
    int64_t ld;
    int m0, M, K, tid;
    bool vec;
    uint32_t r[kPer][4];

    __device__ void init(const uint8_t *slice, int64_t row_stride, int width, int k_len,
                         int col0, bool vec_ok, int t) {
        base = slice;
        ld = row_stride;
        M = width;
        K = k_len;
        m0 = col0;
        vec = vec_ok;
        tid = t;
    }
    __device__ void load(int k0) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int g = tid + T * j;
            const int row = g / (BM / 8), m = m0 + 8 * (g % (BM / 8));
            const int k = k0 + row;
            r[j][0] = r[j][1] = r[j][2] = r[j][3] = 0;
            if ((kGroups % T == 0 || g < kGroups) && k < K && m < M) {
                const uint8_t *ptr = base + (int64_t)k * ld + (int64_t)m * 2;
                if (vec && m + 7 < M) {
                    const uint4 q = *(const uint4 *)ptr;
                    r[j][0] = q.x;
                    r[j][1] = q.y;
                    r[j][2] = q.z;
                    r[j][3] = q.w;
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (m + e < M) r[j][e >> 1] |= ld_u16(ptr + 2 * e) << (16 * (e & 1));
                }
            }
        }
    }
    template <int LD>
    __device__ void store(float (*lds)[LD]) const {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int g = tid + T * j;
            if (!(kGroups % T == 0 || g < kGroups)) continue;
            const int row = g / (BM / 8), c = 8 * (g % (BM / 8));
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t h = (r[j][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                v[e] = BF ? __uint_as_float(h << 16) : half_bits_to_float(h);  // exact
            }
            *(floatx4 *)&lds[row][c] = floatx4{v[0], v[1], v[2], v[3]};
            *(floatx4 *)&lds[row][c + 4] = floatx4{v[4], v[5], v[6], v[7]};
        }
    }
};

// Any block format of block_formats.h: groups of 8 consecutive values of one
// block; fetch in load(), decode in store().
template <class F, int BM, int BK, int T>
struct BlockLoader {
    static constexpr int kGroups = BK * BM / 8;
    static constexpr int kPer = (kGroups + T - 1) / T;
    static_assert(BM % 8 == 0, "tile width must be a multiple of 8");
    const uint8_t *base;
    int64_t ld;
    int m0, M, K, tid;
    uint32_t r[kPer][F::NW];

    __device__ void init(const uint8_t *slice, int64_t row_stride, int width, int k_len,
                         int col0, bool, int t) {
        base = slice;
        ld = row_stride;
        M = width;
        K = k_len;
        m0 = col0;
        tid = t;
    }
    __device__ void load(int k0) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int g = tid + T * j;
            const int row = g / (BM / 8), m = m0 + 8 * (g % (BM / 8));
            const int k = k0 + row;
#pragma unroll
            for (int x = 0; x < F::NW; ++x) r[j][x] = 0;
            if ((kGroups % T == 0 || g < kGroups) && k < K && m < M) {
                const uint8_t *blk = base + (int64_t)k * ld + (int64_t)(m / F::QK) * F::BYTES;
                F::fetch(blk, m % F::QK, r[j]);
            }
        }
    }
    template <int LD>
    __device__ void store(float (*lds)[LD]) const {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int g = tid + T * j;
            if (!(kGroups % T == 0 || g < kGroups)) continue;
            const int row = g / (BM / 8), c = 8 * (g % (BM / 8));
            float v[8];
            F::decode(r[j], (m0 + c) % F::QK, v);
            *(floatx4 *)&lds[row][c] = floatx4{v[0], v[1], v[2], v[3]};
            *(floatx4 *)&lds[row][c + 4] = floatx4{v[4], v[5], v[6], v[7]};
        }
    }
};

template <int AT, int BM, int BK, int T>
struct ALoaderFor;
template <int BM, int BK, int T>
struct ALoaderFor<OUTPROD_TYPE_F32, BM, BK, T> {
    typedef F32Loader<BM, BK, T> type;
};
template <int BM, int BK, int T>
struct ALoaderFor<OUTPROD_TYPE_Q8_0, BM, BK, T> {
    typedef Q8Loader<BM, BK, T> type;
};
template <int BM, int BK, int T>
struct ALoaderFor<OUTPROD_TYPE_Q4_K, BM, BK, T> {
    typedef Q4KLoader<BM, BK, T> type;
};

template <int BM, int BK, int T>
struct ALoaderFor<OUTPROD_TYPE_F16, BM, BK, T> {
    typedef HalfLoader<false, BM, BK, T> type;
};
template <int BM, int BK, int T>
struct ALoaderFor<OUTPROD_TYPE_BF16, BM, BK, T> {
    typedef HalfLoader<true, BM, BK, T> type;
};
#define OUTPROD_BLOCK_LOADER(TYPE, FMT)                  \
    template <int BM, int BK, int T>                     \
    struct ALoaderFor<TYPE, BM, BK, T> {                 \
        typedef BlockLoader<FMT, BM, BK, T> type;        \
    };
OUTPROD_BLOCK_LOADER(OUTPROD_TYPE_Q4_0, FmtQ4_0)
OUTPROD_BLOCK_LOADER(OUTPROD_TYPE_Q4_1, FmtQ4_1)
OUTPROD_BLOCK_LOADER(OUTPROD_TYPE_Q5_0, FmtQ5_0)
OUTPROD_BLOCK_LOADER(OUTPROD_TYPE_Q5_1, FmtQ5_1)
OUTPROD_BLOCK_LOADER(OUTPROD_TYPE_Q2_K, FmtQ2_K)
OUTPROD_BLOCK_LOADER(OUTPROD_TYPE_Q3_K, FmtQ3_K)
OUTPROD_BLOCK_LOADER(OUTPROD_TYPE_Q5_K, FmtQ5_K)
OUTPROD_BLOCK_LOADER(OUTPROD_TYPE_Q6_K, FmtQ6_K)
#undef OUTPROD_BLOCK_LOADER

// ---------------------------------------------------------------- MFMA shapes
// fp32 MFMA, lane l of the wave:
//   32x32x2: supplies A[l%32][k=l/32], B[k=l/32][l%32]; accumulator register r
//            holds D[8*(r/4) + 4*(l/32) + r%4][l%32]            (16 registers)
//   16x16x4: supplies A[l%16][k=l/16], B[k=l/16][l%16]; register r holds
//            D[4*(l/16) + r][l%16]                             (4 registers)
template <int MF>
struct Mfma;
template <>
struct Mfma<32> {
    typedef floatx16 acc_t;
    static constexpr int KS = 2, NR = 16;
    __device__ static acc_t step(float a, float b, acc_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    __device__ static int row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }
};
template <>
struct Mfma<16> {
    typedef floatx4 acc_t;
    static constexpr int KS = 4, NR = 4;
    __device__ static acc_t step(float a, float b, acc_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    __device__ static int row(int r, int lane) { return 4 * (lane >> 4) + r; }
};

// LDS row length: the MF-lane groups of one operand read (rows k, k+1, ...)
// start in different banks.
__host__ __device__ constexpr int lds_ld(int bw, int mf) {
    return bw + (((mf == 32 ? 32 : 16) - bw % 64) % 64 + 64) % 64;
}

// ---------------------------------------------------------------- kernel

template <int AT, int MF, int FM, int FN, int WGM, int WGN, int BK, bool BT>
__global__ __launch_bounds__(64 * WGM * WGN) void tiled_kernel(Problem p0, int tiles_m,
                                                               int tiles_n) {
    typedef Mfma<MF> MM;
    constexpr int T = 64 * WGM * WGN;
    constexpr int WTM = MF * FM, WTN = MF * FN;
    constexpr int BM = WTM * WGM, BN = WTN * WGN;
    constexpr int LDA = lds_ld(BM, MF), LDB = lds_ld(BN, MF);
    constexpr int S = BK / MM::KS;  // MFMA steps per stage
    static_assert(BK % MM::KS == 0 && S % 2 == 0, "stage must hold an even number of MFMA steps");
    __shared__ __attribute__((aligned(16))) float As[2][BK][LDA];
    __shared__ __attribute__((aligned(16))) float Bs[2][BK][LDB];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave % WGM, wn = wave / WGM;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int per_slice = tiles_m * tiles_n;
    // split range outermost, so the tiles of one K range share the XCDs'
    // caches as in an unsplit launch
    const int slices = (int)(p0.ne12 * p0.ne13);
    const int zz = logical / per_slice, rem = logical % per_slice;
    const int z = zz % slices, sp = zz / slices;
    const int m0 = (rem % tiles_m) * BM, n0 = (rem / tiles_m) * BN;
    Problem p = p0;
    SliceBase s = slice_base(p, z);
    if (p.splits > 1) apply_split(p, s, z, sp);
    const int K = (int)p.K, M = (int)p.M, N = (int)p.N;

    typename ALoaderFor<AT, BM, BK, T>::type la;
    typename std::conditional<BT, F32LoaderKT<BN, BK, T>, F32Loader<BN, BK, T>>::type lb;
    la.init(s.a, p.nb01, M, K, m0, p.vec_a, tid);
    lb.init(s.b, BT ? p.nb10 : p.nb11, N, K, n0, p.vec_b, tid);

    typename MM::acc_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < MM::NR; ++r) acc[i][j][r] = 0.f;

    const int ktiles = (K + BK - 1) / BK;
    la.load(0);
    lb.load(0);
    la.store(As[0]);
    lb.store(Bs[0]);
    if (ktiles > 1) {
        la.load(BK);
        lb.load(BK);
    }
    __syncthreads();

    const int kq = lane / MF, col = lane % MF;
    const int a_col = wm * WTM + col, b_col = wn * WTN + col;

    // MFMA steps [s0, s1) of a stage.  Operand fragments are double-buffered
    // in registers: step st+1's LDS reads are issued before step st's MFMAs.
    auto mfma_steps = [&](int cur, int s0, int s1) {
        float af[2][FM], bf[2][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) af[0][i] = As[cur][MM::KS * s0 + kq][a_col + MF * i];
#pragma unroll
        for (int j = 0; j < FN; ++j) bf[0][j] = Bs[cur][MM::KS * s0 + kq][b_col + MF * j];
#pragma unroll
        for (int st = s0; st < s1; ++st) {
            const int x = (st - s0) & 1;
            if (st + 1 < s1) {
                const int kr = MM::KS * (st + 1) + kq;
#pragma unroll
                for (int i = 0; i < FM; ++i) af[x ^ 1][i] = As[cur][kr][a_col + MF * i];
#pragma unroll
                for (int j = 0; j < FN; ++j) bf[x ^ 1][j] = Bs[cur][kr][b_col + MF * j];
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = MM::step(bf[x][j], af[x][i], acc[i][j]);
        }
    };

    for (int t = 0; t < ktiles; ++t) {
        const int cur = t & 1;
        mfma_steps(cur, 0, S / 2);
        if (t + 1 < ktiles) {
            // registers hold stage t+1: decode into the free buffer, then
            // start stage t+2's loads
            la.store(As[cur ^ 1]);
            lb.store(Bs[cur ^ 1]);
            if (t + 2 < ktiles) {
                la.load((t + 2) * BK);
                lb.load((t + 2) * BK);
            }
        }
        mfma_steps(cur, S / 2, S);
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int i0 = m0 + a_col + MF * i;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int r = 0; r < MM::NR; ++r) {
                const int i1 = n0 + wn * WTN + MF * j + MM::row(r, lane);
                if (i0 < M && i1 < N)
                    *(float *)(s.dst + (int64_t)i1 * p.nb1 + (int64_t)i0 * 4) = acc[i][j][r];
            }
        }
    }
}

// ---------------------------------------------------------------- configurations

struct TileCfg {
    int mf, fm, fn, wgm, wgn, bk;
    // Measured rate of the configuration on MI355X (tile area x K per us on
    // the busiest CU, from the q4_K/q8_0 27B-shape sweeps); the planner
    // compares (tiles per CU x tile area) / eff across configurations.
    float eff;
    int bm() const { return mf * fm * wgm; }
    int bn() const { return mf * fn * wgn; }
    int threads() const { return 64 * wgm * wgn; }
};

// 0: 128 x 128, 4 waves of 64 x 64 (32x32x2) -- general purpose
// 1: 160 x 128, 8 waves of 80 x 32 (16x16x4) -- m5120 x n1024 in 256 tiles
// 2: 160 x 64,  4 waves of 80 x 32 (16x16x4) -- m5120 x n1024 in 512 tiles
// 3: 272 x 128, 8 waves of 272 x 16 (16x16x4) -- m17408 x n1024 in 512 tiles
// 4: 64 x 64,   4 waves of 32 x 32 (32x32x2) -- medium problems
// 5: 272 x 64,  4 waves of 272 x 16 (16x16x4) -- m17408 x n1024 in 1024 tiles
// 6: 256 x 128, 8 waves of 64 x 64 (32x32x2)
// 7: 128 x 128, 4 waves of 64 x 64 (32x32x2), 32-row stages
// 8: as 1 with 32-row stages
// 9: as 3 with 32-row stages
constexpr TileCfg kCfgs[] = {
    {32, 2, 2, 2, 2, 16, 12.4f},
    {16, 5, 2, 2, 4, 16, 11.5f},
    {16, 5, 2, 2, 2, 16, 10.4f},
    {16, 17, 1, 1, 8, 16, 12.0f},
    {32, 1, 1, 2, 2, 16, 10.6f},
    {16, 17, 1, 1, 4, 16, 9.8f},
    {32, 2, 2, 4, 2, 16, 12.4f},
    {32, 2, 2, 2, 2, 32, 12.0f},
    {16, 5, 2, 2, 4, 32, 12.2f},
    {16, 17, 1, 1, 8, 32, 12.1f},
};
constexpr int kNumCfgs = sizeof(kCfgs) / sizeof(kCfgs[0]);

template <int AT, int C, bool BT>
const void *cfg_fn() {
    constexpr TileCfg c = kCfgs[C];
    return (const void *)&tiled_kernel<AT, c.mf, c.fm, c.fn, c.wgm, c.wgn, c.bk, BT>;
}

template <int AT, bool BT>
const void *tiled_fn(int variant) {
    switch (variant) {
    case 1: return cfg_fn<AT, 1, BT>();
    case 2: return cfg_fn<AT, 2, BT>();
    case 3: return cfg_fn<AT, 3, BT>();
    case 4: return cfg_fn<AT, 4, BT>();
    case 5: return cfg_fn<AT, 5, BT>();
    case 6: return cfg_fn<AT, 6, BT>();
    case 7: return cfg_fn<AT, 7, BT>();
    case 8: return cfg_fn<AT, 8, BT>();
    case 9: return cfg_fn<AT, 9, BT>();
    default: return cfg_fn<AT, 0, BT>();
    }
}

template <int AT>
const void *tiled_fn(int variant, bool bt) {
    return bt ? tiled_fn<AT, true>(variant) : tiled_fn<AT, false>(variant);
}

// The kernel for a type, configuration and b layout; defined by the
// instantiation files (one per group of a types).  nullptr: type not built.
const void *tiled_kernel_f32(int a_type, int variant, bool bt);
const void *tiled_kernel_half(int a_type, int variant, bool bt);
const void *tiled_kernel_q8(int a_type, int variant, bool bt);
const void *tiled_kernel_q45(int a_type, int variant, bool bt);
const void *tiled_kernel_k4(int a_type, int variant, bool bt);
const void *tiled_kernel_k(int a_type, int variant, bool bt);

}  // namespace tiled
}  // namespace outprod
