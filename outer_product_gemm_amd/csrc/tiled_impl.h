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
// Pipeline (checked loop, run): the registers hold stage t+1 while stage t is
// multiplied; halfway through stage t's MFMAs they are decoded into the other
// LDS buffer and the loads of stage t+2 are issued, so a global load has a
// whole stage of matrix work to arrive.  One barrier per stage.  Full tiles
// of the multi-column tile shapes run run_pipe instead: two raw register
// sets, each stage's decode spread over its MFMA steps.
// b may also have its K dim contiguous (the transposed gradient view of the
// matmul backward); that loader transposes into the same LDS tile, which is
// stored with a column swizzle (b_swizzle).
// MFMA operand roles: A operand (rows) = b values -> dst rows i1;
// B operand (columns) = a values -> dst columns i0, so the lanes of one
// accumulator row write consecutive floats of a dst row.
#pragma once

#include <type_traits>
#include <utility>

#include "block_formats.h"
#include "kernel_common.h"
#include "outprod.h"

namespace outprod {
namespace tiled {

// ---------------------------------------------------------------- loaders
// Each loader moves a BK x BW tile (BW columns of BK consecutive K rows) of
// one operand: load() issues the global reads of a stage into registers,
// store() converts them to fp32 and writes the LDS tile [k][column].
// Work is split into groups (4 floats, or 8 or 16 quantized values); thread
// tid takes groups tid, tid+T, ...; the last round is guarded when T does not
// divide the group count (or, with REDO, repeats a group: group_index).

// f(integral_constant<int, 0>()), ..., f(integral_constant<int, N-1>()):
// a loop whose index is a compile-time constant in the body.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>()), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>());
}

// Group index of a thread's round: group g = tid + T*j.  With REDO (the
// full-tile pipelined loop, which has no branches) a thread past the last
// group of the final round takes a group it already owns, or one another
// thread owns when there are fewer groups than threads: the same loads and
// decode, and its LDS write stores the value that is already there.
template <int G, int T, bool REDO>
__device__ __forceinline__ int group_index(int g) {
    if constexpr (!REDO || G % T == 0)
        return g;
    else if constexpr (G >= T)
        return g < G ? g : g - T;
    else
        return g < G ? g : g % G;
}

// Column swizzle of the b tile in LDS: row k of a tile whose width is a
// multiple of 64 stores column n at n ^ (((k / 4) % 4) * 16), a permutation
// of 16-column blocks within each 64-column group.  The transposing loaders
// then write 4 consecutive k of 16 columns into 64 different banks, and the
// MFMA operand reads (16 or 32 consecutive columns of rows that share k / 4)
// stay contiguous.  Tiles 80 wide are stored unswizzled.
template <int BW>
__device__ __forceinline__ constexpr int b_swizzle(int k) {
    return BW % 64 == 0 ? ((k >> 2) & 3) << 4 : 0;
}

// f32 rows.  SWZ: the tile is b's, stored with b_swizzle.
template <int BW, int BK, int T, bool SWZ = false, bool PRE = false>
struct F32Loader {
    static constexpr int kGroups = BK * BW / 4;
    static constexpr int kPer = (kGroups + T - 1) / T;
    static_assert(BW % 4 == 0, "tile width must be a multiple of 4");
    const uint8_t *base;
    int64_t ld;
    int w0, W, K, tid;
    bool vec;
    floatx4 r[kPer];
    // PRE: each group's byte offset from the slice at k = 0, computed once
    // per tile
    int64_t off[PRE ? kPer : 1];

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
    // PRE: the per-group offsets (called by the threads that run the loads,
    // once per tile, before the first)
    __device__ void pre() {
        if constexpr (PRE) {
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const int g = tid + T * j;
                off[j] = (int64_t)(g / (BW / 4)) * ld + (int64_t)(w0 + 4 * (g % (BW / 4))) * 4;
            }
        }
    }
    // FULL: the whole tile is in range and 16-byte aligned (uniform,
    // checked by the caller): unconditional vector loads.
    template <bool FULL, bool REDO = false>
    __device__ void load(int k0) {
        if constexpr (PRE && FULL && !REDO) {
            const uint8_t *bk = base + (int64_t)k0 * ld;
            static_for<kPer>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                constexpr bool always = kGroups % T == 0 || T * (j + 1) <= kGroups;
                if (always || tid + T * j < kGroups) r[j] = *(const floatx4 *)(bk + off[j]);
            });
            return;
        }
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int g = group_index<kGroups, T, REDO>(tid + T * j);
            const int row = g / (BW / 4), c = w0 + 4 * (g % (BW / 4));
            const int k = k0 + row;
            floatx4 v = {0.f, 0.f, 0.f, 0.f};
            if (FULL) {
                if (REDO || kGroups % T == 0 || g < kGroups)
                    v = *(const floatx4 *)(base + (int64_t)k * ld + (int64_t)c * 4);
            } else if ((REDO || kGroups % T == 0 || g < kGroups) && k < K) {
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
    template <int LD, bool REDO = false, int J0 = 0, int J1 = kPer>
    __device__ void store(float (*lds)[LD]) const {
#pragma unroll
        for (int j = J0; j < J1; ++j) {
            const int g = group_index<kGroups, T, REDO>(tid + T * j);
            if (REDO || kGroups % T == 0 || g < kGroups) {
                const int row = g / (BW / 4), c = 4 * (g % (BW / 4));
                *(floatx4 *)&lds[row][SWZ ? c ^ b_swizzle<BW>(row) : c] = r[j];
            }
        }
    }
};

// f32 b whose K dim is contiguous (a transposed view; column stride `ld`):
// groups of 4 consecutive k of one column, written transposed into the same
// [k][column] LDS tile (with b_swizzle).  Four consecutive groups are the 16
// consecutive k (64 bytes) of one column, so a wave's load covers 16 columns
// in whole 64-byte segments.
template <int BW, int BK, int T>
struct F32LoaderKT {
    static constexpr int kGroups = BK / 4 * BW;
    static constexpr int kPer = (kGroups + T - 1) / T;
    static_assert(BK % 4 == 0, "stage rows must be a multiple of 4");
    static constexpr int KQ = BK / 4 < 4 ? BK / 4 : 4;  // k groups per column segment
    const uint8_t *base;
    int64_t ld;
    int w0, W, K, tid;
    bool vec;
    floatx4 r[kPer];

    // group g -> column n and group of 4 rows kq of the stage
    __device__ static int col_of(int g) { return (g / KQ) % BW; }
    __device__ static int kq_of(int g) { return g % KQ + KQ * (g / (KQ * BW)); }

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
    template <bool FULL, bool REDO = false>
    __device__ void load(int k0) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int g = group_index<kGroups, T, REDO>(tid + T * j);
            const int n = col_of(g), kq = kq_of(g);
            const int c = w0 + n, k = k0 + 4 * kq;
            floatx4 v = {0.f, 0.f, 0.f, 0.f};
            if (FULL) {
                if (REDO || kGroups % T == 0 || g < kGroups)
                    v = *(const floatx4 *)(base + (int64_t)c * ld + (int64_t)k * 4);
            } else if ((REDO || kGroups % T == 0 || g < kGroups) && c < W) {
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
    template <int LD, bool REDO = false, int J0 = 0, int J1 = kPer>
    __device__ void store(float (*lds)[LD]) const {
#pragma unroll
        for (int j = J0; j < J1; ++j) {
            const int g = group_index<kGroups, T, REDO>(tid + T * j);
            if (REDO || kGroups % T == 0 || g < kGroups) {
                const int n = col_of(g), kq = kq_of(g);
                const int sn = n ^ b_swizzle<BW>(4 * kq);
#pragma unroll
                for (int e = 0; e < 4; ++e) lds[4 * kq + e][sn] = r[j][e];
            }
        }
    }
};

// f32 b columns gathered from anywhere (the routed slots of one expert in
// MUL_MAT_ID_BACK): column n of the tile starts at cols[n] (nullptr: no
// column) and holds K contiguous floats; groups of 4 consecutive k written
// transposed into the [k][column] LDS tile (with b_swizzle), four
// consecutive groups covering 16 consecutive k of one column.  vec: every
// column start is 16-byte aligned.
template <int BW, int BK, int T>
struct GatherLoaderKT {
    static constexpr int kGroups = BK / 4 * BW;
    static constexpr int kPer = (kGroups + T - 1) / T;
    static_assert(BK % 4 == 0, "stage rows must be a multiple of 4");
    static constexpr int KQ = BK / 4 < 4 ? BK / 4 : 4;
    const uint8_t *col[kPer];
    int K, tid;
    bool vec;
    floatx4 r[kPer];

    // group g -> column n and group of 4 rows kq (as F32LoaderKT)
    __device__ static int col_of(int g) { return (g / KQ) % BW; }
    __device__ static int kq_of(int g) { return g % KQ + KQ * (g / (KQ * BW)); }

    __device__ void init(const uint8_t *const *cols, int k_len, bool vec_ok, int t) {
        K = k_len;
        vec = vec_ok;
        tid = t;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int g = tid + T * j;
            col[j] = (kGroups % T == 0 || g < kGroups) ? cols[col_of(g)] : nullptr;
        }
    }
    template <bool FULL>
    __device__ void load(int k0) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int g = tid + T * j;
            const int k = k0 + 4 * kq_of(g);
            floatx4 v = {0.f, 0.f, 0.f, 0.f};
            if (FULL) {
                // K in range and 16-byte aligned; columns past the tile's
                // slots (nullptr) stay zero
                if ((kGroups % T == 0 || g < kGroups) && col[j] != nullptr)
                    v = *(const floatx4 *)(col[j] + (int64_t)k * 4);
            } else if (col[j] != nullptr && k < K) {
                const uint8_t *ptr = col[j] + (int64_t)k * 4;
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
                const int n = col_of(g), kq = kq_of(g);
                const int sn = n ^ b_swizzle<BW>(4 * kq);
#pragma unroll
                for (int e = 0; e < 4; ++e) lds[4 * kq + e][sn] = r[j][e];
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
    template <bool FULL, bool REDO = false>
    __device__ void load(int k0) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int g = group_index<kGroups, T, REDO>(tid + T * j);
            const int row = g / (BM / 8), m = m0 + 8 * (g % (BM / 8));
            const int k = k0 + row;
            d[j] = 0;
            q[j][0] = q[j][1] = q[j][2] = q[j][3] = 0;
            if ((REDO || kGroups % T == 0 || g < kGroups) && (FULL || (k < K && m < M))) {
                const uint8_t *blk = base + (int64_t)k * ld + (int64_t)(m >> 5) * 34;
                const uint16_t *qs = (const uint16_t *)(blk + 2 + (m & 31));
                d[j] = *(const uint16_t *)blk;
#pragma unroll
                for (int e = 0; e < 4; ++e) q[j][e] = qs[e];
            }
        }
    }
    template <int LD, bool REDO = false, int J0 = 0, int J1 = kPer>
    __device__ void store(float (*lds)[LD]) const {
#pragma unroll
        for (int j = J0; j < J1; ++j) {
            const int g = group_index<kGroups, T, REDO>(tid + T * j);
            if (!(REDO || kGroups % T == 0 || g < kGroups)) continue;
            const int row = g / (BM / 8), c = 8 * (g % (BM / 8));
            const float dd = half_bits_to_float(d[j]);
            float v[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // value = d * q, exact in fp32 (11 + 7 significant bits); the
                // int8 -> float conversions are single sub-dword instructions
                v[2 * e] = dd * (float)(int8_t)(q[j][e] & 0xFFu);
                v[2 * e + 1] = dd * (float)(int8_t)(q[j][e] >> 8);
            }
            *(floatx4 *)&lds[row][c] = floatx4{v[0], v[1], v[2], v[3]};
            *(floatx4 *)&lds[row][c + 4] = floatx4{v[4], v[5], v[6], v[7]};
        }
    }
};

// q4_K a: groups of GV (8 or 16) consecutive values of one 32-value
// sub-block; a group's scale and min are decoded once for its GV values.
template <int BM, int BK, int T, int GV, bool PRE = false>
struct Q4KLoader {
    static constexpr int kGroups = BK * BM / GV;
    static constexpr int kPer = (kGroups + T - 1) / T;
    static constexpr int NQ = GV / 4;  // code dwords per group
    static_assert(BM % GV == 0 && (GV == 8 || GV == 16), "tile width must be a multiple of the group");
    const uint8_t *base;
    int64_t ld;
    int m0, M, K, tid;
    uint32_t dd[kPer], s0[kPer], s1[kPer], s2[kPer], q[kPer][NQ];
    // PRE: each group's byte offset from the slice at k = 0 (its block
    // header) and its codes' offset within the block, computed once per
    // tile, so a stage's loads cost one 64-bit add per group
    int64_t off[PRE ? kPer : 1];
    int qo[PRE ? kPer : 1];

    __device__ void init(const uint8_t *slice, int64_t row_stride, int width, int k_len,
                         int col0, bool, int t) {
        base = slice;
        ld = row_stride;
        M = width;
        K = k_len;
        m0 = col0;
        tid = t;
    }
    // PRE: the per-group offsets (called by the threads that run the loads,
    // once per tile, before the first)
    __device__ void pre() {
        if constexpr (PRE) {
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const int g = tid + T * j;
                const int row = g / (BM / GV), m = m0 + GV * (g % (BM / GV));
                const int w = m & 255;
                off[j] = (int64_t)row * ld + (int64_t)(m >> 8) * 144;
                qo[j] = 16 + 32 * ((w >> 5) >> 1) + (w & 31);
            }
        }
    }
    template <bool FULL, bool REDO = false>
    __device__ void load(int k0) {
        if constexpr (PRE && FULL && !REDO) {
            // every group of the full rounds is in range: unconditional loads;
            // only the last round's groups past kGroups are skipped
            const uint8_t *bk = base + (int64_t)k0 * ld;
            static_for<kPer>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                constexpr bool always = kGroups % T == 0 || T * (j + 1) <= kGroups;
                if (always || tid + T * j < kGroups) {
                    const uint32_t *hdr = (const uint32_t *)(bk + off[j]);
                    const uint32_t *qs = (const uint32_t *)(bk + off[j] + qo[j]);
                    dd[j] = hdr[0];
                    s0[j] = hdr[1];
                    s1[j] = hdr[2];
                    s2[j] = hdr[3];
#pragma unroll
                    for (int e = 0; e < NQ; ++e) q[j][e] = qs[e];
                }
            });
            return;
        }
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int g = group_index<kGroups, T, REDO>(tid + T * j);
            const int row = g / (BM / GV), m = m0 + GV * (g % (BM / GV));
            const int k = k0 + row;
            dd[j] = s0[j] = s1[j] = s2[j] = 0;
#pragma unroll
            for (int e = 0; e < NQ; ++e) q[j][e] = 0;
            if ((REDO || kGroups % T == 0 || g < kGroups) && (FULL || (k < K && m < M))) {
                const uint8_t *blk = base + (int64_t)k * ld + (int64_t)(m >> 8) * 144;
                const int w = m & 255, sub = w >> 5, pos = w & 31;
                const uint32_t *hdr = (const uint32_t *)blk;
                const uint32_t *qs = (const uint32_t *)(blk + 16 + 32 * (sub >> 1) + pos);
                dd[j] = hdr[0];
                s0[j] = hdr[1];
                s1[j] = hdr[2];
                s2[j] = hdr[3];
#pragma unroll
                for (int e = 0; e < NQ; ++e) q[j][e] = qs[e];
            }
        }
    }
    template <int LD, bool REDO = false, int J0 = 0, int J1 = kPer>
    __device__ void store(float (*lds)[LD]) const {
#pragma unroll
        for (int j = J0; j < J1; ++j) {
            const int g = group_index<kGroups, T, REDO>(tid + T * j);
            if (!(REDO || kGroups % T == 0 || g < kGroups)) continue;
            const int row = g / (BM / GV), c = GV * (g % (BM / GV));
            const int sub = ((m0 + c) & 255) >> 5;
            // 6-bit scale and min of sub-block `sub` from the 12 packed bytes
            // (bytes 0-3 in s0, 4-7 in s1, 8-11 in s2), without branches: for
            // sub < 4 the low 6 bits of bytes sub and 4+sub; otherwise the
            // nibbles of byte 8+(sub-4) below the top two bits of bytes sub-4
            // and sub.  Bit-field extracts with per-lane offsets and widths
            // (the top bits' width is 0 for sub < 4, which extracts 0).
            const uint32_t sh = 8 * (sub & 3);
            const bool hi = sub >= 4;
            const uint32_t w_lo = hi ? 4u : 6u, w_top = hi ? 2u : 0u;
            const uint32_t sc = __builtin_amdgcn_ubfe(hi ? s2[j] : s0[j], sh, w_lo) |
                                (__builtin_amdgcn_ubfe(s0[j], sh + 6, w_top) << 4);
            const uint32_t mn = __builtin_amdgcn_ubfe(hi ? s2[j] : s1[j], hi ? sh + 4 : sh, w_lo) |
                                (__builtin_amdgcn_ubfe(s1[j], sh + 6, w_top) << 4);
            const float d = half_bits_to_float(dd[j] & 0xFFFFu);
            const float dmin = half_bits_to_float(dd[j] >> 16);
            const float ds = d * (float)sc;    // exact: <= 17 significant bits
            const float dm = dmin * (float)mn; // exact
            // this sub-block's nibble of each code byte, as bytes
            const int shift = 4 * (sub & 1);
#pragma unroll
            for (int e = 0; e < NQ; ++e) {
                const uint32_t n = opaque((q[j][e] >> shift) & 0x0F0F0F0Fu);
                // value = d*sc*q - dmin*m: the product is exact, one rounding
                *(floatx4 *)&lds[row][c + 4 * e] =
                    floatx4{ds * (float)(n & 0xFFu) - dm, ds * (float)((n >> 8) & 0xFFu) - dm,
                            ds * (float)((n >> 16) & 0xFFu) - dm, ds * (float)(n >> 24) - dm};
            }
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
    template <bool FULL, bool REDO = false>
    __device__ void load(int k0) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int g = group_index<kGroups, T, REDO>(tid + T * j);
            const int row = g / (BM / 8), m = m0 + 8 * (g % (BM / 8));
            const int k = k0 + row;
            r[j][0] = r[j][1] = r[j][2] = r[j][3] = 0;
            if ((REDO || kGroups % T == 0 || g < kGroups) && (FULL || (k < K && m < M))) {
                const uint8_t *ptr = base + (int64_t)k * ld + (int64_t)m * 2;
                if (FULL || (vec && m + 7 < M)) {
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
    template <int LD, bool REDO = false, int J0 = 0, int J1 = kPer>
    __device__ void store(float (*lds)[LD]) const {
#pragma unroll
        for (int j = J0; j < J1; ++j) {
            const int g = group_index<kGroups, T, REDO>(tid + T * j);
            if (!(REDO || kGroups % T == 0 || g < kGroups)) continue;
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
    template <bool FULL, bool REDO = false>
    __device__ void load(int k0) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int g = group_index<kGroups, T, REDO>(tid + T * j);
            const int row = g / (BM / 8), m = m0 + 8 * (g % (BM / 8));
            const int k = k0 + row;
#pragma unroll
            for (int x = 0; x < F::NW; ++x) r[j][x] = 0;
            if ((REDO || kGroups % T == 0 || g < kGroups) && (FULL || (k < K && m < M))) {
                const uint8_t *blk = base + (int64_t)k * ld + (int64_t)(m / F::QK) * F::BYTES;
                F::fetch(blk, m % F::QK, r[j]);
            }
        }
    }
    template <int LD, bool REDO = false, int J0 = 0, int J1 = kPer>
    __device__ void store(float (*lds)[LD]) const {
#pragma unroll
        for (int j = J0; j < J1; ++j) {
            const int g = group_index<kGroups, T, REDO>(tid + T * j);
            if (!(REDO || kGroups % T == 0 || g < kGroups)) continue;
            const int row = g / (BM / 8), c = 8 * (g % (BM / 8));
            float v[8];
            F::decode(r[j], (m0 + c) % F::QK, v);
            *(floatx4 *)&lds[row][c] = floatx4{v[0], v[1], v[2], v[3]};
            *(floatx4 *)&lds[row][c + 4] = floatx4{v[4], v[5], v[6], v[7]};
        }
    }
};

// Loaders whose decode chunks go on the first MFMA steps of a stage in the
// pipelined loop, so the next stage's loads are issued early: the 2-byte
// aligned K-quant blocks (q3_K, q6_K), which fetch a group with 10-11 16-bit
// loads (m5120 k17408: q6_K 1587 -> 1536 us, q3_K 1616 -> 1578 us; the other
// types ran as fast or slower that way, q8_0 439 -> 467 us at k5120).
template <class L>
struct early_chunks : std::false_type {};
template <int BM, int BK, int T>
struct early_chunks<BlockLoader<FmtQ3_K, BM, BK, T>> : std::true_type {};
template <int BM, int BK, int T>
struct early_chunks<BlockLoader<FmtQ6_K, BM, BK, T>> : std::true_type {};

// a's loader for a type.  WIDE: the tile runs the pipelined full-tile loop,
// where q4_K decodes groups of 16 values (one scale/min decode per 16); the
// checked loop keeps groups of 8, whose tail round is spread more evenly
// over the waves.
// PRE: the loader keeps each group's offsets from one tile's setup (for the
// loader waves, whose stage loop is short of VALU issue; the q4_K and f32
// loaders implement it, the others ignore it).
template <int AT, int BM, int BK, int T, bool WIDE = false, bool PRE = false>
struct ALoaderFor;
template <int BM, int BK, int T, bool WIDE, bool PRE>
struct ALoaderFor<OUTPROD_TYPE_F32, BM, BK, T, WIDE, PRE> {
    typedef F32Loader<BM, BK, T, false, PRE> type;
};
template <int BM, int BK, int T, bool WIDE, bool PRE>
struct ALoaderFor<OUTPROD_TYPE_Q8_0, BM, BK, T, WIDE, PRE> {
    typedef Q8Loader<BM, BK, T> type;
};
template <int BM, int BK, int T, bool WIDE, bool PRE>
struct ALoaderFor<OUTPROD_TYPE_Q4_K, BM, BK, T, WIDE, PRE> {
    typedef Q4KLoader<BM, BK, T, WIDE ? 16 : 8, PRE> type;
};

template <int BM, int BK, int T, bool WIDE, bool PRE>
struct ALoaderFor<OUTPROD_TYPE_F16, BM, BK, T, WIDE, PRE> {
    typedef HalfLoader<false, BM, BK, T> type;
};
template <int BM, int BK, int T, bool WIDE, bool PRE>
struct ALoaderFor<OUTPROD_TYPE_BF16, BM, BK, T, WIDE, PRE> {
    typedef HalfLoader<true, BM, BK, T> type;
};
#define OUTPROD_BLOCK_LOADER(TYPE, FMT)                  \
    template <int BM, int BK, int T, bool WIDE, bool PRE> \
    struct ALoaderFor<TYPE, BM, BK, T, WIDE, PRE> {      \
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

// l.pre() where the loader has it (the loaders that keep per-group offsets).
template <class L>
__device__ __forceinline__ auto loader_pre(L &l, int) -> decltype(l.pre(), void()) {
    l.pre();
}
template <class L>
__device__ __forceinline__ void loader_pre(L &, long) {}

// One workgroup's BM x BN tile: the K loop shared by the OUT_PROD kernel and
// the grouped MUL_MAT_ID_BACK kernel.  WGM x WGN waves, each with FM x FN
// MFMA blocks of MF x MF; BK rows of K per pipeline stage.
template <int MF, int FM, int FN, int WGM, int WGN, int BK>
struct TileCore {
    typedef Mfma<MF> MM;
    typedef typename MM::acc_t acc_t;
    static constexpr int T = 64 * WGM * WGN;
    static constexpr int WTM = MF * FM, WTN = MF * FN;
    static constexpr int BM = WTM * WGM, BN = WTN * WGN;
    static constexpr int LDA = lds_ld(BM, MF), LDB = lds_ld(BN, MF);
    static constexpr int S = BK / MM::KS;  // MFMA steps per stage
    static_assert(BK % MM::KS == 0 && S % 2 == 0, "stage must hold an even number of MFMA steps");

    // acc = the tile's sum over k < K of a-rows x b-rows, from the loaders'
    // stages.  Ends with a barrier (the LDS buffers may be reused).  With
    // PART, a wave runs only its first fn_act (wave-uniform) MFMA blocks along
    // the tile's rows: the rows past them are not needed (a grouped tile
    // holding fewer slots than its height), so those MFMAs are skipped.
    // With DEEP, two register sets of raw operand data: a stage's global
    // loads are issued two stages before its decode into LDS (one stage
    // without), for tiles with too little MFMA work per stage to cover a
    // load's latency in one.
    template <bool FULL, bool PART = false, bool DEEP = false, class LA, class LB>
    __device__ static void run(LA &la, LB &lb, int K, float (&As)[2][BK][LDA],
                               float (&Bs)[2][BK][LDB], acc_t (&acc)[FM][FN], int fn_act = FN) {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int wm = wave % WGM, wn = wave / WGM;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < MM::NR; ++r) acc[i][j][r] = 0.f;

        const int ktiles = (K + BK - 1) / BK;
        LA la1 = la;  // DEEP: the second register set (odd stages)
        LB lb1 = lb;
        la.template load<FULL>(0);
        lb.template load<FULL>(0);
        if (DEEP && ktiles > 1) {
            la1.template load<FULL>(BK);
            lb1.template load<FULL>(BK);
        }
        la.store(As[0]);
        lb.store(Bs[0]);
        if (ktiles > 1 + DEEP) {
            la.template load<FULL>((1 + DEEP) * BK);
            lb.template load<FULL>((1 + DEEP) * BK);
        }
        __syncthreads();

        const int kq = lane / MF, col = lane % MF;
        const int a_col = wm * WTM + col, b_col = wn * WTN + col;

        // MFMA steps [s0, s1) of a stage.  Operand fragments are double-buffered
        // in registers: step st+1's LDS reads are issued before step st's MFMAs.
        // Column-of-waves tiles (WGM == 1: every wave spans the whole i0
        // width, 17 MFMA blocks) raise the wave's priority for its MFMA steps,
        // so a wave ready to feed the matrix core wins issue over one that is
        // decoding: 3.5% faster there, slower for the other tile shapes.
        constexpr bool kPrio = WGM == 1;
        auto mfma_steps = [&](int cur, int s0, int s1) {
            if constexpr (kPrio) __builtin_amdgcn_s_setprio(1);
            float af[2][FM], bf[2][FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) af[0][i] = As[cur][MM::KS * s0 + kq][a_col + MF * i];
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bf[0][j] = Bs[cur][MM::KS * s0 + kq][(b_col + MF * j) ^ b_swizzle<BN>(MM::KS * s0)];
#pragma unroll
            for (int st = s0; st < s1; ++st) {
                const int x = (st - s0) & 1;
                if (st + 1 < s1) {
                    const int kr = MM::KS * (st + 1) + kq;
#pragma unroll
                    for (int i = 0; i < FM; ++i) af[x ^ 1][i] = As[cur][kr][a_col + MF * i];
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        bf[x ^ 1][j] = Bs[cur][kr][(b_col + MF * j) ^ b_swizzle<BN>(MM::KS * (st + 1))];
                }
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        if (!PART || j < fn_act) acc[i][j] = MM::step(bf[x][j], af[x][i], acc[i][j]);
            }
            if constexpr (kPrio) __builtin_amdgcn_s_setprio(0);
        };
        const bool mma = !PART || fn_act > 0;

        if constexpr (!DEEP) {
            for (int t = 0; t < ktiles; ++t) {
                const int cur = t & 1;
                if (mma) mfma_steps(cur, 0, S / 2);
                if (t + 1 < ktiles) {
                    // registers hold stage t+1: decode into the free buffer,
                    // then start stage t+2's loads
                    la.store(As[cur ^ 1]);
                    lb.store(Bs[cur ^ 1]);
                    if (t + 2 < ktiles) {
                        la.template load<FULL>((t + 2) * BK);
                        lb.template load<FULL>((t + 2) * BK);
                    }
                }
                if (mma) mfma_steps(cur, S / 2, S);
                __syncthreads();
            }
        } else {
            // set 0 holds the even stages, set 1 the odd ones: stage t
            // decodes stage t+1's set into the free buffer, then loads stage
            // t+3 into that set
            auto stage = [&](int t, LA &xa, LB &xb) {
                const int cur = t & 1;
                if (mma) mfma_steps(cur, 0, S / 2);
                if (t + 1 < ktiles) {
                    xa.store(As[cur ^ 1]);
                    xb.store(Bs[cur ^ 1]);
                    if (t + 3 < ktiles) {
                        xa.template load<FULL>((t + 3) * BK);
                        xb.template load<FULL>((t + 3) * BK);
                    }
                }
                if (mma) mfma_steps(cur, S / 2, S);
                __syncthreads();
            };
            for (int t = 0; t < ktiles; t += 2) {
                stage(t, la1, lb1);
                if (t + 1 < ktiles) stage(t + 1, la, lb);
            }
        }
    }

    // Full tiles (every load in range, K a whole number of stages): the same
    // contraction as run<true>, summed in the same order, by a stage loop
    // without branches.  Two register sets hold the raw operand data of the
    // next two stages, so a stage's global loads are issued two stages before
    // they are decoded; stage t+1's decode into the free LDS buffer and the
    // loads of stage t+3 are spread over stage t's MFMA steps (one a group
    // per step, then the b tile, then the loads), where the matrix core has
    // work queued while the wave decodes.
    template <class LA, class LB>
    __device__ static void run_pipe(LA (&la)[2], LB (&lb)[2], int K, float (&As)[2][BK][LDA],
                                    float (&Bs)[2][BK][LDB], acc_t (&acc)[FM][FN]) {
        static_assert(LA::kPer + 2 <= S, "a stage has too few MFMA steps for its decode");
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int wm = wave % WGM, wn = wave / WGM;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < MM::NR; ++r) acc[i][j][r] = 0.f;
        const int kq = lane / MF, col = lane % MF;
        const int a_col = wm * WTM + col, b_col = wn * WTN + col;
        // a's last round: when its groups fill whole waves, the waves past
        // them skip it (a scalar branch) instead of decoding a group again
        constexpr int kTailGroups = LA::kGroups - T * (LA::kPer - 1);
        constexpr bool kTailWave = LA::kGroups % T != 0 && kTailGroups % 64 == 0;
        const bool tail_on = __builtin_amdgcn_readfirstlane(wave) * 64 < kTailGroups;

        // One stage: the MFMA steps on LDS buffer `cur`; with DEC, the
        // decode of register set (xa, xb) into buffer cur^1; with LOAD, then
        // the loads of rows [kload, kload + BK) into that set.
        auto stage = [&](auto dec_c, auto load_c, int cur, LA &xa, LB &xb, int kload) {
            constexpr bool DEC = decltype(dec_c)::value, LOAD = decltype(load_c)::value;
            float af[2][FM], bf[2][FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) af[0][i] = As[cur][kq][a_col + MF * i];
#pragma unroll
            for (int j = 0; j < FN; ++j) bf[0][j] = Bs[cur][kq][(b_col + MF * j) ^ b_swizzle<BN>(0)];
            static_for<S>([&](auto st_c) {
                constexpr int st = decltype(st_c)::value, x = st & 1;
                if constexpr (st + 1 < S) {
                    const int kr = MM::KS * (st + 1) + kq;
#pragma unroll
                    for (int i = 0; i < FM; ++i) af[x ^ 1][i] = As[cur][kr][a_col + MF * i];
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        bf[x ^ 1][j] = Bs[cur][kr][(b_col + MF * j) ^ b_swizzle<BN>(MM::KS * (st + 1))];
                }
                auto mfmas = [&]() {
#pragma unroll
                    for (int i = 0; i < FM; ++i)
#pragma unroll
                        for (int j = 0; j < FN; ++j) acc[i][j] = MM::step(bf[x][j], af[x][i], acc[i][j]);
                };
                // chunk c of the decode work (a group c < kPer, then the b
                // tile, then the loads) runs in step c * S / (kPer + 2), or
                // in step c for the formats with early_chunks
                constexpr int NC = LA::kPer + 2;
                constexpr int c = early_chunks<LA>::value ? st : (st * NC + S - 1) / S;
                constexpr bool here = DEC && c < NC && (early_chunks<LA>::value || c * S / NC == st);
                if constexpr (here && c == LA::kPer - 1 && kTailWave) {
                    // the last a round has groups only in the first waves:
                    // a wave-uniform branch, MFMAs on both sides
                    if (tail_on) {
                        mfmas();
                        xa.template store<LDA, true, c, c + 1>(As[cur ^ 1]);
                    } else {
                        mfmas();
                    }
                } else {
                    mfmas();
                    if constexpr (here && c < LA::kPer) {
                        xa.template store<LDA, true, c, c + 1>(As[cur ^ 1]);
                    } else if constexpr (here && c == LA::kPer) {
                        xb.template store<LDB, true>(Bs[cur ^ 1]);
                    } else if constexpr (here && c == LA::kPer + 1 && LOAD) {
                        xa.template load<true, true>(kload);
                        xb.template load<true, true>(kload);
                    }
                }
            });
        };
        typedef std::integral_constant<bool, true> Y;
        typedef std::integral_constant<bool, false> N;

        const int ktiles = K / BK;
        la[0].template load<true, true>(0);
        lb[0].template load<true, true>(0);
        if (ktiles > 1) {
            la[1].template load<true, true>(BK);
            lb[1].template load<true, true>(BK);
        }
        la[0].template store<LDA, true>(As[0]);
        lb[0].template store<LDB, true>(Bs[0]);
        if (ktiles > 2) {
            la[0].template load<true, true>(2 * BK);
            lb[0].template load<true, true>(2 * BK);
        }
        __syncthreads();
        int t = 0;
        // steady state: stage t decodes set 1 (stage t+1) and loads stage t+3
        // into it; stage t+1 decodes set 0 (stage t+2) and loads stage t+4
        for (; t + 4 < ktiles; t += 2) {
            stage(Y(), Y(), 0, la[1], lb[1], (t + 3) * BK);
            __syncthreads();
            stage(Y(), Y(), 1, la[0], lb[0], (t + 4) * BK);
            __syncthreads();
        }
        for (; t < ktiles; ++t) {
            const bool dec = t + 1 < ktiles, ld = t + 3 < ktiles;
            if (t & 1) {
                if (ld) stage(Y(), Y(), 1, la[0], lb[0], (t + 3) * BK);
                else if (dec) stage(Y(), N(), 1, la[0], lb[0], 0);
                else stage(N(), N(), 1, la[0], lb[0], 0);
            } else {
                if (ld) stage(Y(), Y(), 0, la[1], lb[1], (t + 3) * BK);
                else if (dec) stage(Y(), N(), 0, la[1], lb[1], 0);
                else stage(N(), N(), 0, la[1], lb[1], 0);
            }
            __syncthreads();
        }
    }

    // Wave-specialized K loop: the WGM x WGN multiplying waves only read
    // operand fragments from LDS and issue MFMAs; P more waves (threads
    // T .. T + 64P - 1, which own the loaders) load and decode.  Three LDS
    // stages form a ring; the loaders keep D raw register sets.
    // - Loader round r (r = -1, 0, ...) writes stage r + 2 into buffer
    //   (r + 2) % 3, then issues the loads of stage r + 2 + D into the set it
    //   freed, and ends with barrier X_r (the prologue writes stage 0 and
    //   passes one barrier first).
    // - A multiplying wave passes X_{t-1} after the MFMAs of stage t's first
    //   step.  Between X_{t-1} and X_t it reads stages t and t + 1 (buffers
    //   t % 3 and (t + 1) % 3) while the loaders fill (t + 2) % 3, whose
    //   previous stage (t - 1) it finished before X_{t-1}; stage t + 1 was
    //   written before X_{t-1}.
    // - Its fragments are double-buffered across stage boundaries, so the
    //   matrix core has the step's MFMAs queued while the wave waits at a
    //   barrier.  Every wave passes 1 + ktiles barriers.
    // The sum over k has the same order as in run (the MFMA steps in k
    // order), so the result is the same bits.  For the column-of-waves tile
    // this takes the decode off the multiplying waves, whose 68 accumulator
    // registers leave no room for the pipelined loop.  What still costs:
    // with the loaders' decode and LDS writes switched off (builds kept out
    // of the library) the m17408 q4_K launch ran 1292 us instead of 1441
    // us, with the loads alone kept 1287 us.  The loader waves by themselves
    // need 492 us, yet beside the MFMA waves their round is the stage's
    // critical path: sleeps added to it lengthened the launch nearly one for
    // one.  Per-buffer LDS counters polled in place of the barriers ran
    // slower (1476 us).
    template <bool FULL, int P, int D, class LA, class LB>
    __device__ static void run_ws(LA &la, LB &lb, int K, float (&As)[3][BK][LDA],
                                  float (&Bs)[3][BK][LDB], acc_t (&acc)[FM][FN]) {
        const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
        const int ktiles = (K + BK - 1) / BK;
        if (wave >= WGM * WGN) {
            loader_pre(la, 0);
            loader_pre(lb, 0);
            // D register sets: set (s % D) holds stage s from its loads until
            // its decode, D rounds later
            LA la1 = la;
            LB lb1 = lb;
            la.template load<FULL>(0);
            lb.template load<FULL>(0);
            la.store(As[0]);
            lb.store(Bs[0]);
            if (ktiles > 1) {
                (D == 2 ? la1 : la).template load<FULL>(BK);
                (D == 2 ? lb1 : lb).template load<FULL>(BK);
            }
            if (D == 2 && ktiles > 2) {
                la.template load<FULL>(2 * BK);
                lb.template load<FULL>(2 * BK);
            }
            __syncthreads();
            // round r: stage r + 2 into buffer (r + 2) % 3, then the loads
            // of stage r + 2 + D into the set it freed
            auto round = [&](int r, LA &xa, LB &xb) {
                if (r + 2 < ktiles) {
                    const int b = (r + 2) % 3;
                    xa.store(As[b]);
                    xb.store(Bs[b]);
                    if (r + 2 + D < ktiles) {
                        xa.template load<FULL>((r + 2 + D) * BK);
                        xb.template load<FULL>((r + 2 + D) * BK);
                    }
                }
                __syncthreads();
            };
            if constexpr (D == 2) {
                for (int r = -1; r <= ktiles - 2; r += 2) {
                    round(r, la1, lb1);
                    if (r + 1 <= ktiles - 2) round(r + 1, la, lb);
                }
            } else {
                for (int r = -1; r <= ktiles - 2; ++r) round(r, la, lb);
            }
            return;
        }
        const int lane = threadIdx.x & 63;
        const int wm = wave % WGM, wn = wave / WGM;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < MM::NR; ++r) acc[i][j][r] = 0.f;
        const int kq = lane / MF, col = lane % MF;
        const int a_col = wm * WTM + col, b_col = wn * WTN + col;
        float af[2][FM], bf[2][FN];
        auto frag = [&](int buf, int st, float(&xa)[FM], float(&xb)[FN]) {
            const int kr = MM::KS * st + kq;
#pragma unroll
            for (int i = 0; i < FM; ++i) xa[i] = As[buf][kr][a_col + MF * i];
#pragma unroll
            for (int j = 0; j < FN; ++j)
                xb[j] = Bs[buf][kr][(b_col + MF * j) ^ b_swizzle<BN>(MM::KS * st)];
        };
        __syncthreads();
        frag(0, 0, af[0], bf[0]);
        int cur = 0;
        for (int t = 0; t < ktiles; ++t) {
            const int nxt = cur == 2 ? 0 : cur + 1;
            static_for<S>([&](auto st_c) {
                constexpr int st = decltype(st_c)::value, x = st & 1;
                // the next step's fragments (after the last stage: a read of
                // a buffer whose values are not used)
                if constexpr (st + 1 < S)
                    frag(cur, st + 1, af[x ^ 1], bf[x ^ 1]);
                else
                    frag(nxt, 0, af[x ^ 1], bf[x ^ 1]);
                // keep those reads ahead of this step's MFMAs (the scheduler
                // otherwise moves each read next to its use, one wait per
                // MFMA pair)
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j) acc[i][j] = MM::step(bf[x][j], af[x][i], acc[i][j]);
                if constexpr (st == 0) {
                    // the step's MFMAs go out before the barrier's wait
                    __builtin_amdgcn_sched_barrier(0);
                    __syncthreads();
                }
            });
            cur = nxt;
        }
    }

    // Tile-relative dst position of accumulator (i, j, register r) of this
    // lane: column (along i0) and row (along i1).
    __device__ static int col_of(int i) {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        return (wave % WGM) * WTM + lane % MF + MF * i;
    }
    __device__ static int row_of(int j, int r) {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        return (wave / WGM) * WTN + MF * j + MM::row(r, lane);
    }
};

// P > 0: P more waves that load and decode for the multiplying ones (run_ws).
template <int AT, int MF, int FM, int FN, int WGM, int WGN, int BK, bool BT, int P = 0, int D = 1>
__global__ __launch_bounds__(64 * (WGM * WGN + P)) void tiled_kernel(Problem p0, int tiles_m,
                                                                     int tiles_n, int group_m) {
    typedef TileCore<MF, FM, FN, WGM, WGN, BK> C;
    constexpr int T = C::T, BM = C::BM, BN = C::BN;
    constexpr int NS = P > 0 ? 3 : 2;  // LDS stages
    __shared__ __attribute__((aligned(16))) float As[NS][BK][C::LDA];
    __shared__ __attribute__((aligned(16))) float Bs[NS][BK][C::LDB];

    const int tid = threadIdx.x;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int per_slice = tiles_m * tiles_n;
    // split range outermost, so the tiles of one K range share the XCDs'
    // caches as in an unsplit launch
    const int slices = (int)(p0.ne12 * p0.ne13);
    const int zz = logical / per_slice, rem = logical % per_slice;
    const int z = zz % slices, sp = zz / slices;
    // consecutive logical tiles walk groups of group_m m-tiles, i0 fastest
    // within a group (group_m = tiles_m: i0 fastest over the slice; 1: i1
    // fastest); the last group may be narrower
    const int gsize = group_m * tiles_n;
    const int grp = rem / gsize, idx = rem % gsize;
    const int gm = tiles_m - grp * group_m < group_m ? tiles_m - grp * group_m : group_m;
    const int m0 = (grp * group_m + idx % gm) * BM;
    const int n0 = (idx / gm) * BN;
    Problem p = p0;
    SliceBase s = slice_base(p, z);
    if (p.splits > 1) apply_split(p, s, z, sp);
    const int K = (int)p.K, M = (int)p.M, N = (int)p.N;

    // the pipelined loop needs registers for two raw stages next to the
    // accumulators (not the column-of-waves tiles: with 68 accumulator
    // registers per wave they spill) and a step per a group plus two; q4_K
    // takes 16-value groups there when their last round fills whole waves
    constexpr bool kPipeCfg = P == 0 && FM * FN * C::MM::NR <= 64;
    constexpr int kG16 = BK * BM / 16;
    constexpr bool kWide = kPipeCfg && (kG16 % T == 0 || kG16 % T % 64 == 0);
    // threads that run the loaders: all, or the P loader waves
    constexpr int TL = P > 0 ? 64 * P : T;
    const int tl = P > 0 ? tid - T : tid;
    // loader waves: the loaders keep each group's offsets from the tile's
    // setup (PRE; for the other kernels it measured no faster, and slower on
    // the split 64 x 64 tiles of m1536: 59.9 -> 67.3 us)
    typename ALoaderFor<AT, BM, BK, TL, kWide, (P > 0)>::type la;
    typename std::conditional<BT, F32LoaderKT<BN, BK, TL>, F32Loader<BN, BK, TL, true, (P > 0)>>::type lb;
    la.init(s.a, p.nb01, M, K, m0, p.vec_a, tl);
    lb.init(s.b, BT ? p.nb10 : p.nb11, N, K, n0, p.vec_b, tl);

    // whole tile in range, whole stages, 16-byte aligned operands: the loads
    // need no per-lane checks
    const bool a_vec_ok = (AT != OUTPROD_TYPE_F32 && AT != OUTPROD_TYPE_F16 && AT != OUTPROD_TYPE_BF16) ||
                          p.vec_a;
    const bool full = m0 + BM <= M && n0 + BN <= N && K % BK == 0 && a_vec_ok && p.vec_b;
    typename C::acc_t acc[FM][FN];
    typedef decltype(la) LA;
    typedef decltype(lb) LB;
    constexpr bool kPipe = kPipeCfg && LA::kPer + 2 <= C::S;
    if constexpr (P > 0) {
        // two raw register sets do not fit beside q3_K, q5_K and q6_K's
        // groups (they spilled 8-25 registers): one set for those
        constexpr int kD = AT == OUTPROD_TYPE_Q3_K || AT == OUTPROD_TYPE_Q5_K || AT == OUTPROD_TYPE_Q6_K ? 1 : D;
        if (full)
            C::template run_ws<true, P, kD>(la, lb, K, As, Bs, acc);
        else
            C::template run_ws<false, P, kD>(la, lb, K, As, Bs, acc);
        if (tid >= T) return;  // loader waves hold no accumulators
    } else if (full) {
        if constexpr (kPipe) {
            LA la2[2] = {la, la};
            LB lb2[2] = {lb, lb};
            C::run_pipe(la2, lb2, K, As, Bs, acc);
        } else {
            // loads two stages ahead (not q3_K with 32-row stages, whose
            // decode registers leave no room for the second set)
            constexpr bool kDeep = BK == 16 || AT != OUTPROD_TYPE_Q3_K;
            C::template run<true, false, kDeep>(la, lb, K, As, Bs, acc);
        }
    } else {
        C::template run<false>(la, lb, K, As, Bs, acc);
    }

#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int i0 = m0 + C::col_of(i);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int r = 0; r < C::MM::NR; ++r) {
                const int i1 = n0 + C::row_of(j, r);
                if (i0 < M && i1 < N)
                    *(float *)(s.dst + (int64_t)i1 * p.nb1 + (int64_t)i0 * 4) = acc[i][j][r];
            }
        }
    }
}

// Grouped MUL_MAT_ID_BACK: workgroup (tile j of the routing table, m-tile)
// multiplies expert tile_e[j] by the gradient columns of up to BN of its
// routed slots (sorted[offsets[e] + tile_r0[j] + n]) and writes each slot's
// dst row segment.  Workgroups past the table's n_tiles exit at once.
template <int AT, int MF, int FM, int FN, int WGM, int WGN, int BK>
__global__ __launch_bounds__(64 * WGM * WGN) void tiled_id_kernel(IdProblem p, int tiles_m) {
    typedef TileCore<MF, FM, FN, WGM, WGN, BK> C;
    constexpr int T = C::T, BM = C::BM, BN = C::BN;
    __shared__ __attribute__((aligned(16))) float As[2][BK][C::LDA];
    __shared__ __attribute__((aligned(16))) float Bs[2][BK][C::LDB];
    __shared__ const uint8_t *gcol[BN];
    __shared__ uint8_t *drow[BN];

    const int tid = threadIdx.x;
    // The grid is sized for the most tiles any routing can need; only the
    // first tiles_m * n_tiles blocks have work.  The dispatcher deals blocks
    // to the XCDs round-robin, so the working blocks cover every XCD; the
    // remap over exactly those blocks keeps each XCD's tiles contiguous.
    const int *ws = (const int *)p.ws;
    const int real = tiles_m * ws[p.off_ntiles];
    if ((int)blockIdx.x >= real) return;  // uniform: the whole workgroup exits
    const int logical = xcd_remap(blockIdx.x, real);
    const int j = logical / tiles_m, m0 = (logical % tiles_m) * BM;
    const int e = ws[p.off_tile_e + j];
    const int first = ws[p.off_offsets + e] + ws[p.off_tile_r0 + j];
    const int end = ws[p.off_offsets + e + 1];
    const int cnt = end - first < BN ? end - first : BN;
    const int nu = (int)p.n_used;
    for (int n = tid; n < BN; n += T) {
        if (n < cnt) {
            const int slot = ws[p.off_sorted + first + n];
            const int i = slot % nu, t = slot / nu;
            gcol[n] = p.g + (int64_t)i * p.nbg1 + (int64_t)t * p.nbg2;
            drow[n] = p.dst + (int64_t)i * p.nbd1 + (int64_t)t * p.nbd2;
        } else {
            gcol[n] = nullptr;
            drow[n] = nullptr;
        }
    }
    __syncthreads();
    const int K = (int)p.K, M = (int)p.M;

    typename ALoaderFor<AT, BM, BK, T>::type la;
    GatherLoaderKT<BN, BK, T> lb;
    la.init(p.as + (int64_t)e * p.nb02, p.nb01, M, K, m0, p.vec_a, tid);
    lb.init(gcol, K, p.vec_g, tid);

    // waves whose slot rows are all past the expert's last slot skip their MFMAs
    typename C::acc_t acc[FM][FN];
    // MFMA blocks of MF slot rows this wave needs: those holding a slot
    const int wave_row0 = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) / WGM * C::WTN;  // first slot row
    const int need = (cnt - wave_row0 + MF - 1) / MF;
    const int fn_act = need < 0 ? 0 : need > FN ? FN : need;
    const bool a_vec_ok = (AT != OUTPROD_TYPE_F32 && AT != OUTPROD_TYPE_F16 && AT != OUTPROD_TYPE_BF16) ||
                          p.vec_a;
    // the expert's rows and K in range (the slot columns may stop short of
    // BN: the gather loader leaves those zero)
    const bool full = m0 + BM <= M && K % BK == 0 && a_vec_ok && p.vec_g;
    if (full)
        C::template run<true, true, true>(la, lb, K, As, Bs, acc, fn_act);
    else
        C::template run<false, true, true>(la, lb, K, As, Bs, acc, fn_act);

#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int i0 = m0 + C::col_of(i);
#pragma unroll
        for (int jj = 0; jj < FN; ++jj) {
#pragma unroll
            for (int r = 0; r < C::MM::NR; ++r) {
                const int n = C::row_of(jj, r);
                if (i0 < M && n < cnt) *(float *)(drow[n] + (int64_t)i0 * 4) = acc[i][jj][r];
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
    // Loader waves (0: every wave loads, decodes and multiplies; > 0: the
    // wgm x wgn waves only multiply and ws more waves load and decode, with
    // three LDS stages).
    int ws = 0;
    int wsd = 1;  // the loader waves' raw register sets (loads this many stages ahead)
    int bm() const { return mf * fm * wgm; }
    int bn() const { return mf * fn * wgn; }
    int threads() const { return 64 * (wgm * wgn + ws); }
    int stages() const { return ws ? 3 : 2; }
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
// 10: as 2 with 32-row stages
// 11: as 4 with 32-row stages
// 12: 128 x 80, 4 waves of 32 x 80 (16x16x4) -- 80-slot tiles (routed experts)
// 13: 64 x 80,  4 waves of 16 x 80 (16x16x4)
// 14: 80 x 256, 8 waves of 80 x 32 (16x16x4) in one row, 32-row stages --
//     m5120 x n1024 in 256 tiles with half the a decode per flop of 8 (the
//     planner rates it per a type: cfg_eff)
// Grouped MUL_MAT_ID_BACK only (past kNumCfgs): slot tiles that every wave
// spans whole, so in a tile holding an expert's few dozen slots every wave
// skips the same MFMA blocks:
// 15: 128 x 128, 8 waves of 16 x 128 (16x16x4)
// 16: 128 x 128, 4 waves of 32 x 128 (16x16x4)
// 17: 128 x 96,  8 waves of 16 x 96 (16x16x4)
// 18: as 17 with 32-row stages
// (64 x 128 tiles of 4 waves and 32-row stages of 15 ran at half its rate
// on the 64-expert shapes.)
// OUT_PROD, with 8 more waves that only load and decode (run_ws; 1024
// threads, three LDS stages: 156 KB, one workgroup per CU):
// 19: as 9 (272 x 128, 8 multiplying waves of 272 x 16), loads one stage ahead
// 20: as 19 with loads two stages ahead (two raw register sets)
// -- m17408 x n1024.  Measured against 9 at m17408 k5120 n1024 (eager,
// rotating inputs, best of two rounds, us): q4_K 1503 -> 1444, f32 1450 ->
// 1384, f16 1451 -> 1378, bf16 1447 -> 1377, q4_1 1469 -> 1413, q5_1 1483
// -> 1431, q2_K 1497 -> 1446, q3_K 1733 -> 1684, q5_K 1543 -> 1508, q8_0
// 1581 -> 1526 (20), q4_0 1553 -> 1538 (20), q5_0 1608 -> 1601 (20), q6_K
// 1661 -> 1647 (20).  The same split for the 160 x 128 and 80 x 256 tiles
// of m5120 ran no faster than their pipelined loop (f32 1367 -> 1393 us,
// q4_K 1469 -> 1467, q8_0 1469 -> 1684), so it is not in the menu.
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
    {16, 5, 2, 2, 2, 32, 10.3f},
    {32, 1, 1, 2, 2, 32, 10.7f},
    {16, 2, 5, 4, 1, 16, 10.4f},
    {16, 1, 5, 4, 1, 16, 10.0f},
    {16, 5, 2, 1, 8, 32, 12.5f},
    {16, 1, 8, 8, 1, 16, 10.0f},
    {16, 2, 8, 4, 1, 16, 10.0f},
    {16, 1, 6, 8, 1, 16, 10.0f},
    {16, 1, 6, 8, 1, 32, 10.0f},
    {16, 17, 1, 1, 8, 32, 12.6f, 8, 1},
    {16, 17, 1, 1, 8, 32, 12.6f, 8, 2},
};
// The OUT_PROD menu: configurations 0 .. kNumCfgs-1 and the loader-wave ones.
constexpr int kNumCfgs = 15;
constexpr int kNumAllCfgs = sizeof(kCfgs) / sizeof(kCfgs[0]);
__host__ __device__ constexpr bool dense_cfg(int c) {
    return (c >= 0 && c < kNumCfgs) || (c >= 19 && c < kNumAllCfgs);
}

template <int AT, int C, bool BT>
const void *cfg_fn() {
    constexpr TileCfg c = kCfgs[C];
    return (const void *)&tiled_kernel<AT, c.mf, c.fm, c.fn, c.wgm, c.wgn, c.bk, BT, c.ws, c.wsd>;
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
    case 10: return cfg_fn<AT, 10, BT>();
    case 11: return cfg_fn<AT, 11, BT>();
    case 12: return cfg_fn<AT, 12, BT>();
    case 13: return cfg_fn<AT, 13, BT>();
    case 14: return cfg_fn<AT, 14, BT>();
    case 19: return cfg_fn<AT, 19, BT>();
    case 20: return cfg_fn<AT, 20, BT>();
    default: return cfg_fn<AT, 0, BT>();
    }
}

template <int AT>
const void *tiled_fn(int variant, bool bt) {
    return bt ? tiled_fn<AT, true>(variant) : tiled_fn<AT, false>(variant);
}

// Tile configurations the grouped MUL_MAT_ID_BACK kernel is built for
// (indices into kCfgs): 64-, 80- and 128-slot tiles, 16- and 32-row stages.
constexpr int kIdCfgs[] = {2, 4, 1, 0, 8, 10, 11, 12, 13, 15, 16, 17, 18};
constexpr int kNumIdCfgs = sizeof(kIdCfgs) / sizeof(kIdCfgs[0]);

template <int AT, int C>
const void *id_cfg_fn() {
    constexpr TileCfg c = kCfgs[C];
    return (const void *)&tiled_id_kernel<AT, c.mf, c.fm, c.fn, c.wgm, c.wgn, c.bk>;
}

template <int AT>
const void *id_fn(int cfg) {
    switch (cfg) {
    case 2: return id_cfg_fn<AT, 2>();
    case 4: return id_cfg_fn<AT, 4>();
    case 1: return id_cfg_fn<AT, 1>();
    case 0: return id_cfg_fn<AT, 0>();
    case 8: return id_cfg_fn<AT, 8>();
    case 10: return id_cfg_fn<AT, 10>();
    case 11: return id_cfg_fn<AT, 11>();
    case 12: return id_cfg_fn<AT, 12>();
    case 13: return id_cfg_fn<AT, 13>();
    case 15: return id_cfg_fn<AT, 15>();
    case 16: return id_cfg_fn<AT, 16>();
    case 17: return id_cfg_fn<AT, 17>();
    case 18: return id_cfg_fn<AT, 18>();
    default: return nullptr;
    }
}

// The kernel for a type, configuration and b layout (and, with id = true,
// the grouped MUL_MAT_ID_BACK kernel for a type and configuration); defined
// by the instantiation files (one per group of a types).  nullptr: not built.
const void *tiled_kernel_f32(int a_type, int variant, bool bt, bool id = false);
const void *tiled_kernel_half(int a_type, int variant, bool bt, bool id = false);
const void *tiled_kernel_q8(int a_type, int variant, bool bt, bool id = false);
const void *tiled_kernel_q45(int a_type, int variant, bool bt, bool id = false);
const void *tiled_kernel_k4(int a_type, int variant, bool bt, bool id = false);
const void *tiled_kernel_k(int a_type, int variant, bool bt, bool id = false);

}  // namespace tiled
}  // namespace outprod
