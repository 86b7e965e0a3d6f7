// kernel_skinny.hip -- OUT_PROD for f32 a with few output tiles: the LoRA
// parameter gradients of rank 4/8/24 (pages: "metal: OUT_PROD runs batched,
// broadcast and narrow shapes on the GPU", body: the rank gradients at the 4B's
// shapes) and small per-head products such as the delta-net backward (same
// page: 16 value heads over 4 key heads).  The rank-r shapes move b once and
// do a handful of flops per byte, so they are bound by HBM bandwidth and by
// how fast the chip fills with loads; the per-head shapes have too few
// 128 x 128 tiles to occupy 256 CUs.
//
// Decomposition: one workgroup per strip of 16*CW consecutive columns i1 of b
// (16*CW*4 bytes of every row k) and 16*MT consecutive columns i0 of a, in one
// dst slice, all K rows.  Lane l reads CW consecutive floats of row
// k0 + l/16 at column n0 + CW*(l%16) with one vector load, so the 16 lanes of
// a row read one contiguous segment.  Component c of those CW floats is the A
// operand of one v_mfma_f32_16x16x4_f32 (lane l: b[k0 + l/16][n0 + CW*(l%16) + c])
// whose B operand is read straight from a (lane l, block t: a[k0 + l/16][m0 + MT*(l%16) + t],
// so a lane's MT values are one vector load);
// the MFMA performs the k reduction inside the instruction, and accumulator set
// c holds the dst columns n0 + CW*i + c.  The W waves take interleaved 4-row
// steps of K, each wave issuing the loads of U steps together; their partial
// tiles are summed in LDS in wave order, so the result is deterministic and
// every dst element has one writer.  No atomics; a launch split over K ranges
// writes each range's partial tile to the stream's workspace instead of dst,
// and the reduce kernel adds them in range order.
#include "kernel_common.h"
#include "outprod.h"

namespace outprod {
namespace {

template <int CW>
struct VecF;
template <>
struct VecF<2> {
    typedef float type __attribute__((ext_vector_type(2)));
};
template <>
struct VecF<4> {
    typedef float type __attribute__((ext_vector_type(4)));
};

// CW consecutive floats of b at column `col` of one row.  FULL: the whole
// strip is in range and 16-byte aligned, so one vector load; otherwise element
// loads at clamped (in-range) columns, zeroed past the end of the row.
template <int CW, bool FULL>
__device__ __forceinline__ void load_cols(const uint8_t *row, int col, int N, float *out) {
    if constexpr (FULL && CW > 1) {
        const typename VecF<CW>::type v = *(const typename VecF<CW>::type *)(row + (int64_t)col * 4);
#pragma unroll
        for (int c = 0; c < CW; ++c) out[c] = v[c];
    } else {
#pragma unroll
        for (int c = 0; c < CW; ++c) {
            const int cc = col + c < N ? col + c : N - 1;
            const float v = ldf(row + (int64_t)cc * 4);
            out[c] = col + c < N ? v : 0.f;
        }
    }
}

// G consecutive floats of one row of a starting at column i0 (G = 1, 2, 4,
// 6, 8; i0 a multiple of G).  FULL: a's rows are 16-byte aligned and M is a
// multiple of G, so a group is either wholly in range or wholly past the end:
// vector loads (float4 pieces when G % 4 == 0, else float2: the group's start
// is then 8-byte aligned) at the clamped start min(i0, M-G), with no branch
// (callers zero out-of-range values).  Otherwise element loads at clamped
// columns.
template <int G, bool FULL>
__device__ __forceinline__ void load_a_group(const uint8_t *row, int i0, int M, float *out) {
    if constexpr (G > 1 && FULL) {
        const int ic = i0 < M - G ? i0 : M - G;
        constexpr int P = G % 4 == 0 ? 4 : 2;
        const uint8_t *src = row + (int64_t)ic * 4;
#pragma unroll
        for (int h = 0; h < G / P; ++h) {
            const typename VecF<P>::type v = *(const typename VecF<P>::type *)(src + 4 * P * h);
#pragma unroll
            for (int t = 0; t < P; ++t) out[P * h + t] = v[t];
        }
    } else {
#pragma unroll
        for (int t = 0; t < G; ++t) {
            const int ii = i0 + t < M ? i0 + t : M - 1;
            out[t] = ldf(row + (int64_t)ii * 4);
        }
    }
}

// W_ consecutive floats at ptr (16-byte aligned for W_ = 4, 8-byte for 2).
template <int W_>
__device__ __forceinline__ void ld_vec(const uint8_t *ptr, float *out) {
    if constexpr (W_ == 1) {
        out[0] = *(const float *)ptr;
    } else {
        const typename VecF<W_>::type v = *(const typename VecF<W_>::type *)ptr;
#pragma unroll
        for (int c = 0; c < W_; ++c) out[c] = v[c];
    }
}

// The vector path's whole batches: U steps per wave whose rows all lie below
// K.  A lane's row pointers into a and b advance by a fixed stride per step
// (4*W rows), so the batch's loads are issued back to back with one 64-bit
// add each -- no per-load address multiplies, clamps or selects.  G values of
// a per lane (a group wholly in or wholly past the end of a's row: M % G ==
// 0), CW of b.  Returns the first step left to the general loop.  (The 4x4x1
// kernel keeps the general loop: it measured slower with this one.)
template <int G, int CW, int W, int U>
__device__ __forceinline__ int full_batches(const Problem &p, const SliceBase &s, int col, int ia, int wave,
                                            int kk, floatx4 (&acc)[CW][G]) {
    const int M = (int)p.M;
    const int full_steps = (int)(p.K / 4);
    int base = wave;
    if (base + (U - 1) * W >= full_steps) return base;
    const bool a_in = ia < M;
    const int ic = ia < M - G ? ia : M - G;
    const int64_t bstride = (int64_t)(4 * W) * p.nb11, astride = (int64_t)(4 * W) * p.nb01;
    const uint8_t *pb = s.b + (int64_t)(4 * wave + kk) * p.nb11 + (int64_t)col * 4;
    const uint8_t *pa = s.a + (int64_t)(4 * wave + kk) * p.nb01 + (int64_t)ic * 4;
    for (; base + (U - 1) * W < full_steps; base += W * U) {
        float bv[U][CW];
        float av[U][G];
#pragma unroll
        for (int u = 0; u < U; ++u) ld_vec<G>(pa + u * astride, av[u]);
#pragma unroll
        for (int u = 0; u < U; ++u) ld_vec<CW>(pb + u * bstride, bv[u]);
        pa += U * astride;
        pb += U * bstride;
        // keep the batch's loads ahead of every use: the scheduler would
        // otherwise interleave them with the MFMAs, leaving two or three in
        // flight per wave in a kernel bound by HBM latency
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int t = 0; t < G; ++t) av[u][t] = a_in ? av[u][t] : 0.f;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int c = 0; c < CW; ++c)
#pragma unroll
                for (int t = 0; t < G; ++t)
                    acc[c][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(bv[u][c], av[u][t], acc[c][t], 0, 0, 0);
    }
    return base;
}

// The K loop of one wave.  Loads are unconditional (addresses clamped into
// range, out-of-range values replaced by zero afterwards) so that the U steps'
// loads are all in flight before the first MFMA waits on them.
template <int MT, int CW, int W, int U, bool FULL>
__device__ __forceinline__ void column_k_loop(const Problem &p, const SliceBase &s, int n0, int m0,
                                              int wave, int lane, floatx4 (&acc)[CW][MT]) {
    const int K = (int)p.K, M = (int)p.M, N = (int)p.N;
    const int col = n0 + CW * (lane & 15);
    const int kk = lane >> 4;
    // the MT values of a this lane supplies are consecutive: i0 = m0 + MT*(l%16) + t
    const int ia = m0 + MT * (lane & 15);
    bool a_ok[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) a_ok[t] = ia + t < M;
    const int steps = (K + 3) / 4;
    int base = wave;
    if constexpr (FULL) base = full_batches<MT, CW, W, U>(p, s, col, ia, wave, kk, acc);
    for (; base < steps; base += W * U) {
        float bv[U][CW];
        float av[U][MT];
        // a first: its rows are few and cached, so they arrive before b's
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = (base + u * W) * 4 + kk;
            const int kc = k < K ? k : K - 1;
            load_a_group<MT, FULL>(s.a + (int64_t)kc * p.nb01, ia, M, av[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = (base + u * W) * 4 + kk;
            const int kc = k < K ? k : K - 1;
            load_cols<CW, FULL>(s.b + (int64_t)kc * p.nb11, col, N, bv[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool kok = (base + u * W) * 4 + kk < K;
#pragma unroll
            for (int c = 0; c < CW; ++c) bv[u][c] = kok ? bv[u][c] : 0.f;
#pragma unroll
            for (int t = 0; t < MT; ++t) av[u][t] = (kok && a_ok[t]) ? av[u][t] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int c = 0; c < CW; ++c)
#pragma unroll
                for (int t = 0; t < MT; ++t)
                    acc[c][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(bv[u][c], av[u][t], acc[c][t], 0, 0, 0);
    }
}

// b with its K dim contiguous (a transposed view, column stride nb10), CW = 1:
// lane l reads the 4 consecutive rows kb = k0 + 4*(l/16) .. kb+3 of column
// n0 + l%16 with one 16-byte load.  Component e is the A operand of MFMA step
// e, whose rows are kb + e across the four lane groups (an MFMA's k set need
// not be contiguous; its B operand uses the same rows).  A super-step covers
// 16 rows; the W waves take interleaved super-steps, U of them per batch.
template <int MT, int W, int U, bool FULL>
__device__ __forceinline__ void column_k_loop_kt(const Problem &p, const SliceBase &s, int n0, int m0,
                                                 int wave, int lane, floatx4 (&acc)[1][MT]) {
    const int K = (int)p.K, M = (int)p.M, N = (int)p.N;
    const int col = n0 + (lane & 15);
    const int kq = lane >> 4;
    const uint8_t *bcol = s.b + (int64_t)(col < N ? col : N - 1) * p.nb10;
    const int ia = m0 + MT * (lane & 15);
    bool a_ok[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) a_ok[t] = ia + t < M;
    const int ssteps = (K + 15) / 16;
    for (int base = wave; base < ssteps; base += W * U) {
        float bv[U][4];
        float av[U][4][MT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kb = (base + u * W) * 16 + 4 * kq;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int kc = kb + e < K ? kb + e : K - 1;
                load_a_group<MT, FULL>(s.a + (int64_t)kc * p.nb01, ia, M, av[u][e]);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kb = (base + u * W) * 16 + 4 * kq;
            if constexpr (FULL) {
                const int kc = kb < K ? kb : K - 4;  // K % 16 == 0 on this path
                const floatx4 v = *(const floatx4 *)(bcol + (int64_t)kc * 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) bv[u][e] = v[e];
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int kc = kb + e < K ? kb + e : K - 1;
                    bv[u][e] = ldf(bcol + (int64_t)kc * 4);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kb = (base + u * W) * 16 + 4 * kq;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool kok = kb + e < K;
                bv[u][e] = (kok && col < N) ? bv[u][e] : 0.f;
#pragma unroll
                for (int t = 0; t < MT; ++t) av[u][e][t] = (kok && a_ok[t]) ? av[u][e][t] : 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int t = 0; t < MT; ++t)
                    acc[0][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(bv[u][e], av[u][e][t], acc[0][t], 0, 0, 0);
    }
}

// MT: 16-column blocks of a; CW: columns of b per lane; W: waves; U: 4-row
// steps per wave whose loads are issued together.
template <int MT, int CW, int W, int U>
__global__ __launch_bounds__(64 * W) void skinny_kernel(Problem p0, int col_blocks, int m_blocks) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int n0 = (logical % col_blocks) * (16 * CW);
    const int rest = logical / col_blocks;
    const int m0 = (rest % m_blocks) * 16 * MT;
    const int slices = (int)(p0.ne12 * p0.ne13);
    const int zz = rest / m_blocks;
    const int z = zz % slices, sp = zz / slices;  // split range outermost
    Problem p = p0;
    SliceBase s = slice_base(p, z);
    if (p.splits > 1) apply_split(p, s, z, sp);
    const int M = (int)p.M, N = (int)p.N;

    floatx4 acc[CW][MT];
#pragma unroll
    for (int c = 0; c < CW; ++c)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[c][t] = floatx4{0.f, 0.f, 0.f, 0.f};

    // whole b strip in range, 16-byte aligned rows of a and b (host-checked)
    // and M a multiple of the a group: vector loads without branches
    if (p.b_kt) {
        // K-contiguous b: CW == 1 configurations only (the planner enforces it);
        // a super-step is 16 rows, so U/4 of them per batch
        if constexpr (CW == 1) {
            if (p.vec_b && p.vec_a && n0 + 16 <= N && M % MT == 0 && p.K % 16 == 0)
                column_k_loop_kt<MT, W, (U >= 4 ? U / 4 : 1), true>(p, s, n0, m0, wave, lane, acc);
            else
                column_k_loop_kt<MT, W, (U >= 4 ? U / 4 : 1), false>(p, s, n0, m0, wave, lane, acc);
        }
    } else if (p.vec_b && p.vec_a && n0 + 16 * CW <= N && M % MT == 0) {
        column_k_loop<MT, CW, W, U, true>(p, s, n0, m0, wave, lane, acc);
    } else {
        column_k_loop<MT, CW, W, U, false>(p, s, n0, m0, wave, lane, acc);
    }

    // Sum the W partial tiles in wave order.  In accumulator set (c, t), lane l
    // holds rows i = 4*(l/16) + r (dst column i1 = n0 + CW*i + c) and column
    // j = l%16 (i0 = m0 + MT*j + t).
    __shared__ float red[W][CW][MT][4][64];
#pragma unroll
    for (int c = 0; c < CW; ++c)
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave][c][t][r][lane] = acc[c][t][r];
    __syncthreads();
    for (int o = threadIdx.x; o < 256 * CW * MT; o += 64 * W) {
        const int l = o & 63, r = (o >> 6) & 3, ct = o >> 8;
        const int t = ct % MT, c = ct / MT;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) sum += red[w][c][t][r][l];
        const int i1 = n0 + CW * (4 * (l >> 4) + r) + c;
        const int i0 = m0 + MT * (l & 15) + t;
        if (i1 < N && i0 < M) *(float *)(s.dst + (int64_t)i1 * p.nb1 + (int64_t)i0 * p.nb0) = sum;
    }
}

// ---------------------------------------------------------------- narrow a
// For ne00 <= 32 the 16-block v_mfma_f32_4x4x1_f32 wastes less than a
// 16x16x4 padded to 16 columns of a.  Its lanes 4q'..4q'+3 form block q':
// lane 4q'+i supplies row i of the block's A and column i of its B, and
// accumulator register r of lane 4q'+j holds D[r][j].  With the same b loads
// as above (lane l: row k0 + l/16, columns n0 + CW*(l%16) + c), block
// q' = l/4 covers row k0 + q'/4 and the four b columns n0 + CW*(4*(q'%4) + i) + c;
// in instruction t its B operand is a[k0 + l/16][m0 + T4*(l%4) + t].  So one instruction per
// component c and per 4 columns of a adds a 4 x 4 outer product for each of
// the 4 rows, and the four blocks that share a column group (lanes l, l+16,
// l+32, l+48) hold partial sums over interleaved rows; they are summed with
// the waves in the LDS reduction.
template <int T4, int CW, int W, int U, bool FULL>
__device__ __forceinline__ void narrow_k_loop(const Problem &p, const SliceBase &s, int n0, int m0,
                                              int wave, int lane, floatx4 (&acc)[CW][T4]) {
    const int K = (int)p.K, M = (int)p.M, N = (int)p.N;
    const int col = n0 + CW * (lane & 15);
    const int kk = lane >> 4;
    // the T4 values of a this lane supplies are consecutive: i0 = m0 + T4*(l%4) + t
    const int ia = m0 + T4 * (lane & 3);
    bool a_ok[T4];
#pragma unroll
    for (int t = 0; t < T4; ++t) a_ok[t] = ia + t < M;
    const int steps = (K + 3) / 4;
    for (int base = wave; base < steps; base += W * U) {
        float bv[U][CW];
        float av[U][T4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = (base + u * W) * 4 + kk;
            const int kc = k < K ? k : K - 1;
            load_a_group<T4, FULL>(s.a + (int64_t)kc * p.nb01, ia, M, av[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = (base + u * W) * 4 + kk;
            const int kc = k < K ? k : K - 1;
            load_cols<CW, FULL>(s.b + (int64_t)kc * p.nb11, col, N, bv[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool kok = (base + u * W) * 4 + kk < K;
#pragma unroll
            for (int c = 0; c < CW; ++c) bv[u][c] = kok ? bv[u][c] : 0.f;
#pragma unroll
            for (int t = 0; t < T4; ++t) av[u][t] = (kok && a_ok[t]) ? av[u][t] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int c = 0; c < CW; ++c)
#pragma unroll
                for (int t = 0; t < T4; ++t)
                    acc[c][t] = __builtin_amdgcn_mfma_f32_4x4x1f32(bv[u][c], av[u][t], acc[c][t], 0, 0, 0);
    }
}

// K-contiguous b for the narrow kernel (CW = 1), with the same 16-row
// super-steps as column_k_loop_kt.
template <int T4, int W, int U, bool FULL>
__device__ __forceinline__ void narrow_k_loop_kt(const Problem &p, const SliceBase &s, int n0, int m0,
                                                 int wave, int lane, floatx4 (&acc)[1][T4]) {
    const int K = (int)p.K, M = (int)p.M, N = (int)p.N;
    const int col = n0 + (lane & 15);
    const int kq = lane >> 4;
    const uint8_t *bcol = s.b + (int64_t)(col < N ? col : N - 1) * p.nb10;
    const int ia = m0 + T4 * (lane & 3);
    bool a_ok[T4];
#pragma unroll
    for (int t = 0; t < T4; ++t) a_ok[t] = ia + t < M;
    const int ssteps = (K + 15) / 16;
    for (int base = wave; base < ssteps; base += W * U) {
        float bv[U][4];
        float av[U][4][T4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kb = (base + u * W) * 16 + 4 * kq;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int kc = kb + e < K ? kb + e : K - 1;
                load_a_group<T4, FULL>(s.a + (int64_t)kc * p.nb01, ia, M, av[u][e]);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kb = (base + u * W) * 16 + 4 * kq;
            if constexpr (FULL) {
                const int kc = kb < K ? kb : K - 4;
                const floatx4 v = *(const floatx4 *)(bcol + (int64_t)kc * 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) bv[u][e] = v[e];
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int kc = kb + e < K ? kb + e : K - 1;
                    bv[u][e] = ldf(bcol + (int64_t)kc * 4);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kb = (base + u * W) * 16 + 4 * kq;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool kok = kb + e < K;
                bv[u][e] = (kok && col < N) ? bv[u][e] : 0.f;
#pragma unroll
                for (int t = 0; t < T4; ++t) av[u][e][t] = (kok && a_ok[t]) ? av[u][e][t] : 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int t = 0; t < T4; ++t)
                    acc[0][t] = __builtin_amdgcn_mfma_f32_4x4x1f32(bv[u][e], av[u][e][t], acc[0][t], 0, 0, 0);
    }
}

// T4: 4-column blocks of a (4*T4 columns per workgroup); CW, W, U as above.
template <int T4, int CW, int W, int U>
__global__ __launch_bounds__(64 * W) void narrow_kernel(Problem p0, int col_blocks, int m_blocks) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int n0 = (logical % col_blocks) * (16 * CW);
    const int rest = logical / col_blocks;
    const int m0 = (rest % m_blocks) * 4 * T4;
    const int slices = (int)(p0.ne12 * p0.ne13);
    const int zz = rest / m_blocks;
    const int z = zz % slices, sp = zz / slices;  // split range outermost
    Problem p = p0;
    SliceBase s = slice_base(p, z);
    if (p.splits > 1) apply_split(p, s, z, sp);
    const int M = (int)p.M, N = (int)p.N;

    floatx4 acc[CW][T4];
#pragma unroll
    for (int c = 0; c < CW; ++c)
#pragma unroll
        for (int t = 0; t < T4; ++t) acc[c][t] = floatx4{0.f, 0.f, 0.f, 0.f};

    if (p.b_kt) {
        if constexpr (CW == 1) {
            if (p.vec_b && p.vec_a && n0 + 16 <= N && M % T4 == 0 && p.K % 16 == 0)
                narrow_k_loop_kt<T4, W, (U >= 4 ? U / 4 : 1), true>(p, s, n0, m0, wave, lane, acc);
            else
                narrow_k_loop_kt<T4, W, (U >= 4 ? U / 4 : 1), false>(p, s, n0, m0, wave, lane, acc);
        }
    } else if (p.vec_b && p.vec_a && n0 + 16 * CW <= N && M % T4 == 0) {
        narrow_k_loop<T4, CW, W, U, true>(p, s, n0, m0, wave, lane, acc);
    } else {
        narrow_k_loop<T4, CW, W, U, false>(p, s, n0, m0, wave, lane, acc);
    }

    // Register r of lane l in set (c, t): dst column i1 = n0 + CW*(4*((l/4)%4) + r) + c,
    // i0 = m0 + T4*(l%4) + t, partial over rows k = l/16 (mod 4) of this wave.
    // Sum over the W waves and the 4 lane groups l/16, in that fixed order.
    __shared__ float red[W][CW][T4][4][64];
#pragma unroll
    for (int c = 0; c < CW; ++c)
#pragma unroll
        for (int t = 0; t < T4; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave][c][t][r][lane] = acc[c][t][r];
    __syncthreads();
    // outputs: (c, t, r, l16) with l16 = lane % 16 -> 64 * CW * T4 of them
    for (int o = threadIdx.x; o < 64 * CW * T4; o += 64 * W) {
        const int l16 = o & 15, r = (o >> 4) & 3, ct = o >> 6;
        const int t = ct % T4, c = ct / T4;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w)
#pragma unroll
            for (int g = 0; g < 4; ++g) sum += red[w][c][t][r][l16 + 16 * g];
        const int i1 = n0 + CW * (4 * (l16 >> 2) + r) + c;
        const int i0 = m0 + T4 * (l16 & 3) + t;
        if (i1 < N && i0 < M) *(float *)(s.dst + (int64_t)i1 * p.nb1 + (int64_t)i0 * p.nb0) = sum;
    }
}

struct ColCfg {
    int mma, cw, waves, unroll;  // mma: 16 = 16x16x4 kernel, 4 = 4x4x1 kernel
};
// 16x16x4: 0: 16-col strips, 8 waves x 8 steps   1: 32-col, 8 x 8   2: 64-col, 8 x 8
//          3: 32-col, 16 x 8   4: 64-col, 8 x 16   5: 16-col, 16 x 8
//          11: 32-col, 8 x 16  12: 16-col, 8 x 16
// 4x4x1:   6: 16-col, 8 x 16   7: 32-col, 8 x 16   8: 64-col, 8 x 16
//          9: 32-col, 8 x 8    10: 64-col, 8 x 8
// (8 waves x 16 steps x 4 rows: K = 512 in a single batch of loads per wave)
constexpr ColCfg kColCfgs[] = {{16, 1, 8, 8}, {16, 2, 8, 8},  {16, 4, 8, 8},  {16, 2, 16, 8},
                               {16, 4, 8, 16}, {16, 1, 16, 8}, {4, 1, 8, 16},  {4, 2, 8, 16},
                               {4, 4, 8, 16},  {4, 2, 8, 8},   {4, 4, 8, 8},   {16, 2, 8, 16},
                               {16, 1, 8, 16}};
constexpr int kNumColCfgs = sizeof(kColCfgs) / sizeof(kColCfgs[0]);

template <int MT, int C>
const void *col_fn() {
    constexpr ColCfg c = kColCfgs[C];
    return (const void *)&skinny_kernel<MT, c.cw, c.waves, c.unroll>;
}

template <int MT>
const void *col_fn(int c) {
    switch (c) {
    case 1: return col_fn<MT, 1>();
    case 2: return col_fn<MT, 2>();
    case 3: return col_fn<MT, 3>();
    case 4: return col_fn<MT, 4>();
    case 5: return col_fn<MT, 5>();
    case 11: return col_fn<MT, 11>();
    case 12: return col_fn<MT, 12>();
    default: return col_fn<MT, 0>();
    }
}

template <int T4, int C>
const void *narrow_fn() {
    constexpr ColCfg c = kColCfgs[C];
    return (const void *)&narrow_kernel<T4, c.cw, c.waves, c.unroll>;
}

template <int T4>
const void *narrow_fn(int c) {
    if constexpr (T4 > 4) {
        // wide blocks of a only with strips of up to 32 columns (the LDS
        // reduction of 64-column strips would exceed 160 KB)
        switch (c) {
        case 7: return narrow_fn<T4, 7>();
        case 9: return narrow_fn<T4, 9>();
        default: return narrow_fn<T4, 6>();
        }
    } else {
        switch (c) {
        case 7: return narrow_fn<T4, 7>();
        case 8: return narrow_fn<T4, 8>();
        case 9: return narrow_fn<T4, 9>();
        case 10: return narrow_fn<T4, 10>();
        default: return narrow_fn<T4, 6>();
        }
    }
}

// 4-column blocks of a per workgroup for the narrow kernel: an a up to 32
// columns wide in one i0 block (rank 24 as 6 blocks, not 2 x 4 with 8
// columns of padding); 64-column strips (cw 4) take at most 16 columns per
// block, wider a in several i0 blocks.
int narrow_t4(int64_t M, int cw) {
    return M <= 4 ? 1 : M <= 8 ? 2 : (M <= 16 || cw > 2) ? 4 : M <= 24 ? 6 : 8;
}

const void *narrow_dispatch(int t4, int c) {
    switch (t4) {
    case 1: return narrow_fn<1>(c);
    case 2: return narrow_fn<2>(c);
    case 4: return narrow_fn<4>(c);
    case 6: return narrow_fn<6>(c);
    default: return narrow_fn<8>(c);
    }
}

}  // namespace

// Split count for a column launch of `grid` workgroups: when the strips
// alone leave three quarters of the CUs idle (64 workgroups or fewer), split
// K into ranges of at least 256 rows until the launch has about 256
// workgroups (the partial tiles are small: M x N floats per range).  Measured
// on MI355X: rank-8 gradients with K = 9216 / 17408 over 512 / 1024 columns
// (32 / 64 strips) run 3x faster split; at 80 strips and K = 1024 the extra
// reduce launch costs more than the split gains.
int column_splits(const Problem &p, int64_t grid) {
    if (grid > 64) return 1;
    int64_t s = (256 + grid - 1) / grid;
    if (s > p.K / 256) s = p.K / 256;
    if (s > 64) s = 64;
    while (s > 1 && split_bytes(p, (int)s) > kWorkspaceBytes) --s;
    return s < 1 ? 1 : (int)s;
}

// l->variant on entry: forced configuration + 1, or 0 for automatic;
// l->splits on entry: forced split count, or 0 for automatic.  On return:
// the configuration index (the i0 block width is tile_m) and the split.
bool plan_skinny(const Problem &p, Launch *l) {
    if (p.a_type != OUTPROD_TYPE_F32 || p.M < 1) return false;
    int cfg;
    if (l->variant > 0) {
        if (l->variant > kNumColCfgs) return false;
        cfg = l->variant - 1;
    } else {
        // measured on MI355X with HBM-resident (cache-cold) inputs, ranks
        // 4-32, K = 512 / 1024: b up to 4096 columns wide needs 16-column
        // strips for enough workgroups; up to 16384 columns, 256-byte row
        // segments (64-column strips) read fastest; wider b, and a with
        // several 32-column blocks (per-head products), run 32-column strips.
        // The 4x4x1 kernel is a few % faster for ranks <= 4 over 256-byte
        // segments and slower everywhere else.  K-contiguous b (one column
        // per lane) runs 16 waves of 16x16x4 with 8-step batches: at the
        // split counts the planner picks, 3-17% faster than 8 waves of
        // 4x4x1 or 16x16x4 for ranks 4-24, K 4096-17408 (LoRA dh: 4B
        // 13.7 -> 11.3 us, 27B 27.3 -> 23.7 us).
        if (p.b_kt)
            cfg = 5;
        else if (p.M > 32)
            cfg = 1;
        else if (p.N <= 4096)
            cfg = 0;
        else if (p.N <= 16384)
            cfg = p.M <= 4 ? 10 : 2;
        else
            cfg = 1;
    }
    if (p.b_kt && kColCfgs[cfg].cw != 1) return false;  // forced wide-strip configuration
    const ColCfg &c = kColCfgs[cfg];
    const int cols = 16 * c.cw;
    const int64_t col_blocks = (p.N + cols - 1) / cols;
    int tile_m;
    if (c.mma == 4) {
        tile_m = 4 * narrow_t4(p.M, c.cw);
    } else {
        tile_m = p.M > 16 ? 32 : 16;
    }
    const int64_t m_blocks = (p.M + tile_m - 1) / tile_m;
    l->kernel = OUTPROD_KERNEL_SKINNY;
    l->variant = cfg;
    l->tile_m = tile_m;
    l->tile_n = cols;
    l->tile_k = 4;
    l->block = 64 * c.waves;
    l->lds_bytes = c.waves * c.cw * (c.mma == 4 ? tile_m / 4 : tile_m / 16) * 256 * 4;
    const int64_t grid = col_blocks * m_blocks * p.ne12 * p.ne13;
    int splits = l->splits;
    int64_t ksplit = p.K;
    if (splits > 0) {  // forced: even ranges of any row count
        if (splits > p.K || (splits > 1 && split_bytes(p, splits) > kWorkspaceBytes)) return false;
        if (splits > 1) ksplit = (p.K + splits - 1) / splits;
    } else {
        splits = column_splits(p, grid);
        if (splits > 1) ksplit = split_rows(p.K, splits);
    }
    if (splits > 1) splits = (int)((p.K + ksplit - 1) / ksplit);
    l->splits = splits > 1 ? splits : 1;
    l->ksplit = splits > 1 ? ksplit : p.K;
    l->grid = grid * l->splits;
    return true;
}

hipError_t launch_skinny(const Problem &p, const Launch &l, hipStream_t s) {
    int col_blocks = (int)((p.N + l.tile_n - 1) / l.tile_n);
    int m_blocks = (int)((p.M + l.tile_m - 1) / l.tile_m);
    Problem pp = p;
    void *args[] = {&pp, &col_blocks, &m_blocks};
    const void *fn;
    if (kColCfgs[l.variant].mma == 4)
        fn = narrow_dispatch(l.tile_m / 4, l.variant);
    else
        fn = l.tile_m == 32 ? col_fn<2>(l.variant) : col_fn<1>(l.variant);
    return hipLaunchKernel(fn, dim3((unsigned)l.grid), dim3(l.block), args, 0, s);
}

}  // namespace outprod
