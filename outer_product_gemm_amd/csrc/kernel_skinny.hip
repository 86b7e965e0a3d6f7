// kernel_skinny.hip -- OUT_PROD for f32 a with few output tiles: the LoRA
// parameter gradients of rank 4/8/24 (pages: "metal: OUT_PROD runs batched,
// broadcast and narrow shapes on the GPU", body: the rank gradients at the 4B's
// shapes) and small per-head products such as the delta-net backward (same
// page: 16 value heads over 4 key heads).  The rank-r shapes move b once and
// do a handful of flops per byte, so they are bound by HBM bandwidth and by
// how fast the chip fills with loads; the per-head shapes have too few
// 128 x 128 tiles to occupy 256 CUs.
//
// Decomposition: one workgroup per 16 consecutive columns i1 of b (64 bytes of
// every row k) and 16*MT consecutive columns i0 of a, in one dst slice, all K
// rows.  Its W waves take interleaved 4-row steps of K.  Each step is one
// v_mfma_f32_16x16x4_f32 per 16 columns of a, whose A operand is read
// straight from b (lane l: b[k0 + l/16][n0 + l%16]) and whose B operand is
// read straight from a (lane l: a[k0 + l/16][m0 + 16t + l%16]); the MFMA
// performs the k reduction inside the instruction.  The W per-wave partial
// tiles are then summed in LDS in wave order, so the result is deterministic
// and every dst element has one writer.  No workspace, no atomics.
#include "kernel_common.h"
#include "outprod.h"

namespace outprod {
namespace {

constexpr int kSkinnyCols = 16;  // columns i1 per workgroup

// MT: 16-column blocks of a per workgroup; W: waves; U: 4-row steps per wave
// whose loads are issued together.
template <int MT, int W, int U>
__global__ __launch_bounds__(64 * W) void skinny_kernel(Problem p, int col_blocks, int m_blocks) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int n0 = (logical % col_blocks) * kSkinnyCols;
    const int rest = logical / col_blocks;
    const int m0 = (rest % m_blocks) * 16 * MT;
    const int z = rest / m_blocks;
    const SliceBase s = slice_base(p, z);

    const int K = (int)p.K, M = (int)p.M;
    const int col = n0 + (lane & 15);
    const int kk = lane >> 4;
    const bool col_ok = col < p.N;
    const uint8_t *bcol = s.b + (int64_t)col * 4;
    const uint8_t *acol[MT];
    bool a_ok[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const int i0 = m0 + 16 * t + (lane & 15);
        a_ok[t] = i0 < M;
        acol[t] = s.a + (int64_t)i0 * 4;
    }

    floatx4 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int steps = (K + 3) / 4;
    for (int base = wave; base < steps; base += W * U) {
        float bv[U];
        float av[U][MT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = (base + u * W) * 4 + kk;
            const bool kok = k < K;
            bv[u] = (kok && col_ok) ? ldf(bcol + (int64_t)k * p.nb11) : 0.f;
#pragma unroll
            for (int t = 0; t < MT; ++t)
                av[u][t] = (kok && a_ok[t]) ? ldf(acol[t] + (int64_t)k * p.nb01) : 0.f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int t = 0; t < MT; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(bv[u], av[u][t], acc[t], 0, 0, 0);
    }

    // Sum the W partial tiles in wave order.  Lane l of a wave holds rows
    // 4*(l/16) + r (columns i1) and column l%16 (i0 within block t).
    __shared__ float red[W][MT][4][64];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][t][r][lane] = acc[t][r];
    __syncthreads();
    for (int o = threadIdx.x; o < 256 * MT; o += 64 * W) {
        const int t = o >> 8, r = (o >> 6) & 3, l = o & 63;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) sum += red[w][t][r][l];
        const int i1 = n0 + 4 * (l >> 4) + r;
        const int i0 = m0 + 16 * t + (l & 15);
        if (i1 < p.N && i0 < M) *(float *)(s.dst + (int64_t)i1 * p.nb1 + (int64_t)i0 * 4) = sum;
    }
}

struct ColCfg {
    int waves, unroll;
};
// 0: 8 waves x 8 steps; 1: 16 x 8; 2: 4 x 16; 3: 16 x 4; 4: 8 x 16
constexpr ColCfg kColCfgs[] = {{8, 8}, {16, 8}, {4, 16}, {16, 4}, {8, 16}};
constexpr int kNumColCfgs = sizeof(kColCfgs) / sizeof(kColCfgs[0]);

template <int MT, int C>
const void *col_fn() {
    return (const void *)&skinny_kernel<MT, kColCfgs[C].waves, kColCfgs[C].unroll>;
}

template <int MT>
const void *col_fn(int c) {
    switch (c) {
    case 1: return col_fn<MT, 1>();
    case 2: return col_fn<MT, 2>();
    case 3: return col_fn<MT, 3>();
    case 4: return col_fn<MT, 4>();
    default: return col_fn<MT, 0>();
    }
}

}  // namespace

// l->variant on entry: forced configuration + 1, or 0 for automatic.  On
// return: the configuration index (the i0 block width is tile_m).
bool plan_skinny(const Problem &p, Launch *l) {
    if (p.a_type != OUTPROD_TYPE_F32 || p.M < 1) return false;
    int cfg = 0;
    if (l->variant > 0) {
        if (l->variant > kNumColCfgs) return false;
        cfg = l->variant - 1;
    }
    const int64_t col_blocks = (p.N + kSkinnyCols - 1) / kSkinnyCols;
    const int mt = p.M > 16 ? 2 : 1;
    const int64_t m_blocks = (p.M + 16 * mt - 1) / (16 * mt);
    l->kernel = OUTPROD_KERNEL_SKINNY;
    l->variant = cfg;
    l->tile_m = 16 * mt;
    l->tile_n = kSkinnyCols;
    l->tile_k = 4;
    l->block = 64 * kColCfgs[cfg].waves;
    l->lds_bytes = kColCfgs[cfg].waves * mt * 256 * 4;
    l->grid = col_blocks * m_blocks * p.ne12 * p.ne13;
    return true;
}

hipError_t launch_skinny(const Problem &p, const Launch &l, hipStream_t s) {
    int col_blocks = (int)((p.N + kSkinnyCols - 1) / kSkinnyCols);
    int m_blocks = (int)((p.M + l.tile_m - 1) / l.tile_m);
    Problem pp = p;
    void *args[] = {&pp, &col_blocks, &m_blocks};
    const void *fn = l.tile_m == 32 ? col_fn<2>(l.variant) : col_fn<1>(l.variant);
    return hipLaunchKernel(fn, dim3((unsigned)l.grid), dim3(l.block), args, 0, s);
}

}  // namespace outprod
