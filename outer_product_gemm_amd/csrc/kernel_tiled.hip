// kernel_tiled.hip -- OUT_PROD for wide problems: the grouped-head broadcast
// backward and frozen quantized weight x f32 gradient products (pages: "metal:
// OUT_PROD runs batched, broadcast and narrow shapes on the GPU" -- every
// (i2, i3) slice in one launch instead of one encode per slice; "metal:
// OUT_PROD multiplies in float staging" -- fp32 staging of both operands; and
// the MUL_MAT_ID_BACK page's note that quantized rows are dequantized in
// registers rather than copied).
//
// In BLAS terms each slice is dst(N x M, row-major) = B^T A with A = a's
// [K][M] rows and B = b's [K][N] rows: both operands are K-major, so a K-tile
// of either is BK contiguous row segments.  A workgroup owns a BM x BN dst
// tile (BM along i0, BN along i1) of one slice and walks K in BK-row stages:
//   global -> registers (a: f32 copy or q8_0/q4_K block decode to fp32;
//   b: f32) -> LDS [k][i0] / [k][i1] (fp32, double buffered) ->
//   v_mfma_f32_32x32x2_f32 with fp32 accumulators.
// The next stage's global loads are issued before the current stage's MFMAs
// so their latency hides behind matrix work; one barrier per stage.
// MFMA operand roles: A operand (rows) = b values -> dst rows i1;
// B operand (columns) = a values -> dst columns i0, so the lanes of a
// 32-wide accumulator column write 32 consecutive floats of a dst row.
#include "kernel_common.h"
#include "outprod.h"

namespace outprod {
namespace {

// ---------------------------------------------------------------- loaders

// f32 K-major operand (a or b): BK x BW tile as float4 groups.
template <int BW, int BK, int T>
struct F32Loader {
    static constexpr int kGroups = BK * BW / 4 / T;
    static_assert(kGroups * 4 * T == BK * BW, "tile must split evenly into float4 groups");
    const uint8_t *base;  // slice base + column offset of this thread's groups
    int64_t ld;           // row stride in bytes
    int w0;               // first column of the tile
    int W;                // operand width (M or N)
    int K;
    bool vec;
    int tid;
    floatx4 r[kGroups];

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
        for (int j = 0; j < kGroups; ++j) {
            const int g = tid + T * j;
            const int row = g / (BW / 4), c = w0 + 4 * (g % (BW / 4));
            const int k = k0 + row;
            const uint8_t *ptr = base + (int64_t)k * ld + (int64_t)c * 4;
            floatx4 v = {0.f, 0.f, 0.f, 0.f};
            if (k < K) {
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
        for (int j = 0; j < kGroups; ++j) {
            const int g = tid + T * j;
            const int row = g / (BW / 4), c = 4 * (g % (BW / 4));
            *(floatx4 *)&lds[row][c] = r[j];
        }
    }
};

// q8_0 a: groups of 8 consecutive values of one block.  34-byte blocks are
// only 2-byte aligned, so bytes come in as 16-bit loads.
template <int BM, int BK, int T>
struct Q8Loader {
    static constexpr int kGroups = BK * BM / 8 / T;
    static_assert(kGroups * 8 * T == BK * BM, "tile must split evenly into 8-value groups");
    const uint8_t *base;
    int64_t ld;
    int m0, M, K, tid;
    uint32_t d[kGroups];
    uint32_t q[kGroups][4];

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
        for (int j = 0; j < kGroups; ++j) {
            const int g = tid + T * j;
            const int row = g / (BM / 8), m = m0 + 8 * (g % (BM / 8));
            const int k = k0 + row;
            d[j] = 0;
            q[j][0] = q[j][1] = q[j][2] = q[j][3] = 0;
            if (k < K && m < M) {
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
        for (int j = 0; j < kGroups; ++j) {
            const int g = tid + T * j;
            const int row = g / (BM / 8), c = 8 * (g % (BM / 8));
            const float dd = half_bits_to_float(d[j]);
            floatx4 lo, hi;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // value = d * q, exact in fp32 (11 + 7 significant bits)
                const float q0 = (float)(int8_t)(q[j][e] & 0xFFu);
                const float q1 = (float)(int8_t)(q[j][e] >> 8);
                if (e < 2) {
                    lo[2 * e] = dd * q0;
                    lo[2 * e + 1] = dd * q1;
                } else {
                    hi[2 * e - 4] = dd * q0;
                    hi[2 * e - 3] = dd * q1;
                }
            }
            *(floatx4 *)&lds[row][c] = lo;
            *(floatx4 *)&lds[row][c + 4] = hi;
        }
    }
};

// q4_K a: groups of 8 consecutive values of one 32-value sub-block.
template <int BM, int BK, int T>
struct Q4KLoader {
    static constexpr int kGroups = BK * BM / 8 / T;
    static_assert(kGroups * 8 * T == BK * BM, "tile must split evenly into 8-value groups");
    const uint8_t *base;
    int64_t ld;
    int m0, M, K, tid;
    uint32_t dd[kGroups], s0[kGroups], s1[kGroups], s2[kGroups], q0[kGroups], q1[kGroups];

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
        for (int j = 0; j < kGroups; ++j) {
            const int g = tid + T * j;
            const int row = g / (BM / 8), m = m0 + 8 * (g % (BM / 8));
            const int k = k0 + row;
            dd[j] = s0[j] = s1[j] = s2[j] = q0[j] = q1[j] = 0;
            if (k < K && m < M) {
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
        for (int j = 0; j < kGroups; ++j) {
            const int g = tid + T * j;
            const int row = g / (BM / 8), c = 8 * (g % (BM / 8));
            const int sub = ((m0 + c) & 255) >> 5;
            // 6-bit scale and min of sub-block `sub` from the 12 packed bytes
            // (bytes 0-3 in s0, 4-7 in s1, 8-11 in s2).
            uint32_t sc, mn;
            if (sub < 4) {
                sc = (s0[j] >> (8 * sub)) & 0x3Fu;
                mn = (s1[j] >> (8 * sub)) & 0x3Fu;
            } else {
                const int sh = 8 * (sub - 4);
                const uint32_t lo = (s2[j] >> sh) & 0xFFu;
                sc = (lo & 0x0Fu) | (((s0[j] >> sh) >> 6 & 0x3u) << 4);
                mn = (lo >> 4) | (((s1[j] >> sh) >> 6 & 0x3u) << 4);
            }
            const float d = half_bits_to_float(dd[j] & 0xFFFFu);
            const float dmin = half_bits_to_float(dd[j] >> 16);
            const float ds = d * (float)sc;    // exact: <= 17 significant bits
            const float dm = dmin * (float)mn; // exact
            const int shift = (sub & 1) ? 4 : 0;
            floatx4 lo4, hi4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // value = d*sc*q - dmin*m: the product is exact, one rounding
                lo4[e] = ds * (float)((q0[j] >> (8 * e + shift)) & 0xFu) - dm;
                hi4[e] = ds * (float)((q1[j] >> (8 * e + shift)) & 0xFu) - dm;
            }
            *(floatx4 *)&lds[row][c] = lo4;
            *(floatx4 *)&lds[row][c + 4] = hi4;
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

// ---------------------------------------------------------------- kernel

template <int AT, int BM, int BN, int BK, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) void tiled_kernel(Problem p, int tiles_m,
                                                               int tiles_n) {
    constexpr int T = 64 * WGM * WGN;
    constexpr int WTM = BM / WGM, WTN = BN / WGN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int LDA = BM + 32, LDB = BN + 32;  // +32 floats: the two half-waves
                                                 // of an operand read use other banks
    static_assert(FM * 32 == WTM && FN * 32 == WTN, "wave tile must be 32-aligned");
    static_assert(BK % 2 == 0, "BK must be even");
    __shared__ __attribute__((aligned(16))) float As[2][BK][LDA];
    __shared__ __attribute__((aligned(16))) float Bs[2][BK][LDB];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave % WGM, wn = wave / WGM;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int per_slice = tiles_m * tiles_n;
    const int z = logical / per_slice, rem = logical % per_slice;
    const int m0 = (rem % tiles_m) * BM, n0 = (rem / tiles_m) * BN;
    const SliceBase s = slice_base(p, z);
    const int K = (int)p.K, M = (int)p.M, N = (int)p.N;

    typename ALoaderFor<AT, BM, BK, T>::type la;
    F32Loader<BN, BK, T> lb;
    la.init(s.a, p.nb01, M, K, m0, p.vec_a, tid);
    lb.init(s.b, p.nb11, N, K, n0, p.vec_b, tid);

    floatx16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int ktiles = (K + BK - 1) / BK;
    la.load(0);
    lb.load(0);
    la.store(As[0]);
    lb.store(Bs[0]);
    __syncthreads();

    const int half = lane >> 5, col = lane & 31;
    for (int t = 0; t < ktiles; ++t) {
        const int cur = t & 1;
        const bool more = t + 1 < ktiles;
        if (more) {
            la.load((t + 1) * BK);
            lb.load((t + 1) * BK);
        }
#pragma unroll
        for (int kp = 0; kp < BK / 2; ++kp) {
            const int kr = 2 * kp + half;
            float af[FM], bf[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) af[i] = As[cur][kr][wm * WTM + 32 * i + col];
#pragma unroll
            for (int j = 0; j < FN; ++j) bf[j] = Bs[cur][kr][wn * WTN + 32 * j + col];
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(bf[j], af[i], acc[i][j], 0, 0, 0);
        }
        if (more) {
            la.store(As[cur ^ 1]);
            lb.store(Bs[cur ^ 1]);
        }
        __syncthreads();
    }

    // Accumulator register r of lane l: row 8*(r/4) + 4*(l/32) + r%4 (i1),
    // column l%32 (i0) of the 32x32 block.
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int i0 = m0 + wm * WTM + 32 * i + col;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i1 = n0 + wn * WTN + 32 * j + 8 * (r >> 2) + 4 * half + (r & 3);
                if (i0 < M && i1 < N)
                    *(float *)(s.dst + (int64_t)i1 * p.nb1 + (int64_t)i0 * 4) = acc[i][j][r];
            }
        }
    }
}

// Tile configurations.
struct TileCfg {
    int bm, bn, bk, wgm, wgn;
};
constexpr TileCfg kCfg0 = {128, 128, 16, 2, 2};

template <int AT>
const void *tiled_fn(int variant) {
    (void)variant;
    return (const void *)&tiled_kernel<AT, kCfg0.bm, kCfg0.bn, kCfg0.bk, kCfg0.wgm, kCfg0.wgn>;
}

}  // namespace

bool plan_tiled(const Problem &p, Launch *l) {
    const TileCfg c = kCfg0;
    const int64_t tm = (p.M + c.bm - 1) / c.bm, tn = (p.N + c.bn - 1) / c.bn;
    l->kernel = OUTPROD_KERNEL_TILED;
    l->variant = 0;
    l->tile_m = c.bm;
    l->tile_n = c.bn;
    l->tile_k = c.bk;
    l->block = 64 * c.wgm * c.wgn;
    l->lds_bytes = 2 * c.bk * ((c.bm + 32) + (c.bn + 32)) * 4;
    l->grid = tm * tn * p.ne12 * p.ne13;
    return true;
}

hipError_t launch_tiled(const Problem &p, const Launch &l, hipStream_t s) {
    int tiles_m = (int)((p.M + l.tile_m - 1) / l.tile_m);
    int tiles_n = (int)((p.N + l.tile_n - 1) / l.tile_n);
    Problem pp = p;
    void *args[] = {&pp, &tiles_m, &tiles_n};
    const void *fn;
    switch (p.a_type) {
    case OUTPROD_TYPE_F32: fn = tiled_fn<OUTPROD_TYPE_F32>(l.variant); break;
    case OUTPROD_TYPE_Q8_0: fn = tiled_fn<OUTPROD_TYPE_Q8_0>(l.variant); break;
    case OUTPROD_TYPE_Q4_K: fn = tiled_fn<OUTPROD_TYPE_Q4_K>(l.variant); break;
    default: return hipErrorInvalidValue;
    }
    return hipLaunchKernel(fn, dim3((unsigned)l.grid), dim3(l.block), args, 0, s);
}

}  // namespace outprod
