// kernel_id_back.hip -- MUL_MAT_ID_BACK: the input gradient of MUL_MAT_ID
// through frozen experts, dst row (i, t) = expert ids[i,t] x g[:, i, t]
// (pages: the MUL_MAT_ID_BACK Metal-kernel page: one writer per dst
// element, the expert's rows walked, no expert copied or transposed, the
// frozen-weight types of out_prod decoded in registers).
//
// The page runs one threadgroup per routed slot, so every slot reads its
// expert's whole matrix.  Here the slots are grouped by expert on the device
// and each expert runs as one OUT_PROD-shaped tile job with the slots'
// gradient columns gathered as its b (K contiguous) -- the tiled MFMA kernel
// reads each expert once per 64 or 128 of its slots:
//   1. id_rank_kernel   (one block per 1024 slots) the stable rank of each
//      slot among the block's slots of the same expert (wave ballots), and
//      the block's per-expert counts;
//   2. id_scan_kernel   (one block) per-block bases, per-expert offsets and
//      the tile table (expert, first row) of BN-slot tiles;
//   3. id_place_kernel  the expert-sorted slot list; a slot whose id is not
//      an expert gets a NaN dst row;
//   4. tiled_id_kernel  (tiled_impl.h) one workgroup per (tile, m-tile).
// Up to kIdRouteFused slots, one block does 1-3 in a single launch
// (id_route_kernel), ranking the slots within their experts with LDS
// atomics; the three kernels keep the slots' order within an expert.
// Every dst row has one writer and its sum runs over K in a fixed order
// whatever tile holds its slot: the result is deterministic.  The
// tables live in the stream's workspace; nothing is cleared in advance (every
// entry read is written first, in stream order).
#include <algorithm>
#include <cmath>

#include "kernel_common.h"
#include "outprod.h"
#include "tiled_impl.h"

namespace outprod {
namespace {

__global__ __launch_bounds__(kIdRankBlock) void id_rank_kernel(IdProblem p) {
    constexpr int W = kIdRankBlock / 64;
    __shared__ int wcnt[W][kIdMaxExperts];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int E = (int)p.n_expert, nu = (int)p.n_used;
    const int total = (int)(p.n_used * p.n_tokens);
    int *ws = (int *)p.ws;
    for (int x = tid; x < W * kIdMaxExperts; x += kIdRankBlock) wcnt[x / kIdMaxExperts][x % kIdMaxExperts] = 0;
    __syncthreads();

    const int s = blockIdx.x * kIdRankBlock + tid;
    int e = -1;
    if (s < total) {
        const int i = s % nu, t = s / nu;
        const int v = *(const int *)(p.ids + (int64_t)i * 4 + (int64_t)t * p.nbi1);
        e = (v >= 0 && v < E) ? v : -1;
    }
    // rank among this wave's lower lanes with the same expert: one ballot per
    // distinct expert of the wave (wave-uniform loop)
    int rank = 0;
    unsigned long long todo = __ballot(e >= 0);
    while (todo) {
        const int leader = __ffsll((unsigned long long)todo) - 1;
        const int le = __builtin_amdgcn_readlane(e, leader);
        const unsigned long long peers = __ballot(e == le);
        if (e == le) rank = __popcll(peers & ((1ull << lane) - 1ull));
        if (lane == leader) wcnt[wave][le] = __popcll(peers);
        todo &= ~peers;
    }
    __syncthreads();
    // per expert: exclusive prefix over the waves; the block's count to hist
    for (int x = tid; x < E; x += kIdRankBlock) {
        int acc = 0;
        for (int w = 0; w < W; ++w) {
            const int c = wcnt[w][x];
            wcnt[w][x] = acc;
            acc += c;
        }
        ws[p.off_hist + (int64_t)blockIdx.x * E + x] = acc;
    }
    __syncthreads();
    if (s < total) ws[p.off_rank + s] = e >= 0 ? wcnt[wave][e] + rank : -1;
}

__global__ __launch_bounds__(1024) void id_scan_kernel(IdProblem p) {
    __shared__ int sc[1024], st[1024];
    const int tid = threadIdx.x, E = (int)p.n_expert, B = p.rank_blocks;
    int *ws = (int *)p.ws;
    // per expert: exclusive scan over the rank blocks (hist becomes each
    // block's base within the expert)
    int c = 0;
    if (tid < E) {
        for (int b = 0; b < B; ++b) {
            int *h = ws + p.off_hist + (int64_t)b * E + tid;
            const int v = *h;
            *h = c;
            c += v;
        }
    }
    const int nt = tid < E ? (c + p.bn - 1) / p.bn : 0;
    // inclusive scans over experts of slot counts and tile counts
    sc[tid] = c;
    st[tid] = nt;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int a = tid >= off ? sc[tid - off] : 0;
        const int b = tid >= off ? st[tid - off] : 0;
        __syncthreads();
        sc[tid] += a;
        st[tid] += b;
        __syncthreads();
    }
    if (tid < E) {
        ws[p.off_offsets + tid] = sc[tid] - c;
        const int t0 = st[tid] - nt;
        for (int j = 0; j < nt; ++j) {
            ws[p.off_tile_e + t0 + j] = tid;
            ws[p.off_tile_r0 + t0 + j] = j * p.bn;
        }
    }
    if (tid == E - 1) {
        ws[p.off_offsets + E] = sc[tid];
        ws[p.off_ntiles] = st[tid];
    }
}

__global__ __launch_bounds__(256) void id_place_kernel(IdProblem p) {
    const int s = blockIdx.x * 256 + threadIdx.x;
    const int total = (int)(p.n_used * p.n_tokens), nu = (int)p.n_used, E = (int)p.n_expert;
    if (s >= total) return;
    int *ws = (int *)p.ws;
    const int i = s % nu, t = s / nu;
    const int r = ws[p.off_rank + s];
    if (r < 0) {  // id outside [0, n_expert): the row is NaN
        float *d = (float *)(p.dst + (int64_t)i * p.nbd1 + (int64_t)t * p.nbd2);
        for (int c = 0; c < (int)p.M; ++c) d[c] = __builtin_nanf("");
        return;
    }
    const int e = *(const int *)(p.ids + (int64_t)i * 4 + (int64_t)t * p.nbi1);
    const int blk = s / kIdRankBlock;
    const int pos = ws[p.off_offsets + e] + ws[p.off_hist + (int64_t)blk * E + e] + r;
    ws[p.off_sorted + pos] = s;
}

// Steps 1-3 in one block of 1024 threads for at most kIdRouteFused slots:
// the same per-expert offsets and tile table as the three kernels, and a
// sorted list that holds each expert's slots in an order set by LDS atomics
// (which tile a slot lands in changes no value: a dst row's sum depends
// only on its own gradient column and the expert).  Thread t holds slots
// t, t + 1024, ..., t + 1024 (R - 1) in registers, their ids loaded at once
// (R: the launch's slot count over 1024, rounded up to a power of two).
// One wave scans the per-expert counts 64 experts at a time with lane
// shuffles (no block barriers inside the scan).
template <int R>
__global__ __launch_bounds__(1024) void id_route_kernel(IdProblem p) {
    __shared__ int cnt[kIdMaxExperts];  // slots per expert, then the expert's offset
    const int tid = threadIdx.x, lane = tid & 63;
    const int E = (int)p.n_expert, nu = (int)p.n_used;
    const int total = (int)(p.n_used * p.n_tokens);
    int *ws = (int *)p.ws;
    int ev[R], rk[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int s = r * 1024 + tid;
        ev[r] = -1;
        if (s < total) {
            const int i = s % nu, t = s / nu;
            const int v = *(const int *)(p.ids + (int64_t)i * 4 + (int64_t)t * p.nbi1);
            ev[r] = (v >= 0 && v < E) ? v : -1;
        }
    }
    for (int x = tid; x < E; x += 1024) cnt[x] = 0;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r) rk[r] = ev[r] >= 0 ? atomicAdd(&cnt[ev[r]], 1) : -1;
    __syncthreads();
    // per-expert offsets and the tile table (as id_scan_kernel), by wave 0:
    // an inclusive scan over each run of 64 experts, plus the runs before
    if (tid < 64) {
        int carry_c = 0, carry_t = 0;
        for (int base = 0; base < E; base += 64) {
            const int x = base + lane;
            const int c = x < E ? cnt[x] : 0;
            const int nt = (c + p.bn - 1) / p.bn;
            int ic = c, it = nt;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int a = __shfl_up(ic, off), b = __shfl_up(it, off);
                if (lane >= off) {
                    ic += a;
                    it += b;
                }
            }
            if (x < E) {
                const int o = carry_c + ic - c, t0 = carry_t + it - nt;
                cnt[x] = o;
                ws[p.off_offsets + x] = o;
                for (int j = 0; j < nt; ++j) {
                    ws[p.off_tile_e + t0 + j] = x;
                    ws[p.off_tile_r0 + t0 + j] = j * p.bn;
                }
            }
            carry_c += __shfl(ic, 63);
            carry_t += __shfl(it, 63);
        }
        if (lane == 0) {
            ws[p.off_offsets + E] = carry_c;
            ws[p.off_ntiles] = carry_t;
        }
    }
    __syncthreads();
    // the sorted list (as id_place_kernel)
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int s = r * 1024 + tid;
        if (s >= total) continue;
        if (rk[r] >= 0) {
            ws[p.off_sorted + cnt[ev[r]] + rk[r]] = s;
        } else {  // id outside [0, n_expert): the row is NaN
            const int i = s % nu, t = s / nu;
            float *d = (float *)(p.dst + (int64_t)i * p.nbd1 + (int64_t)t * p.nbd2);
            for (int m = 0; m < (int)p.M; ++m) d[m] = __builtin_nanf("");
        }
    }
}

// The routing kernel for a slot count (at most kIdRouteFused).
const void *id_route_for(int64_t slots) {
    static_assert(kIdRouteFused == 16 * 1024, "instantiations cover 1 to 16 rounds");
    if (slots <= 1024) return (const void *)&id_route_kernel<1>;
    if (slots <= 2048) return (const void *)&id_route_kernel<2>;
    if (slots <= 4096) return (const void *)&id_route_kernel<4>;
    if (slots <= 8192) return (const void *)&id_route_kernel<8>;
    return (const void *)&id_route_kernel<16>;
}

const void *id_kernel_for(int a_type, int cfg) {
    using namespace tiled;
    switch (a_type) {
    case OUTPROD_TYPE_F32: return tiled_kernel_f32(a_type, cfg, false, true);
    case OUTPROD_TYPE_F16:
    case OUTPROD_TYPE_BF16: return tiled_kernel_half(a_type, cfg, false, true);
    case OUTPROD_TYPE_Q8_0:
    case OUTPROD_TYPE_Q4_0:
    case OUTPROD_TYPE_Q4_1: return tiled_kernel_q8(a_type, cfg, false, true);
    case OUTPROD_TYPE_Q5_0:
    case OUTPROD_TYPE_Q5_1: return tiled_kernel_q45(a_type, cfg, false, true);
    case OUTPROD_TYPE_Q4_K:
    case OUTPROD_TYPE_Q2_K: return tiled_kernel_k4(a_type, cfg, false, true);
    case OUTPROD_TYPE_Q3_K:
    case OUTPROD_TYPE_Q5_K:
    case OUTPROD_TYPE_Q6_K: return tiled_kernel_k(a_type, cfg, false, true);
    default: return nullptr;
    }
}

void set_layout(IdProblem &p, int bn) {
    const int64_t slots = p.n_used * p.n_tokens;
    p.bn = bn;
    p.rank_blocks = (int)((slots + kIdRankBlock - 1) / kIdRankBlock);
    p.max_tiles = (int)((slots + bn - 1) / bn + p.n_expert);
    p.off_rank = 0;
    p.off_hist = slots;
    p.off_offsets = p.off_hist + (int64_t)p.rank_blocks * p.n_expert;
    p.off_sorted = p.off_offsets + p.n_expert + 1;
    p.off_tile_e = p.off_sorted + slots;
    p.off_tile_r0 = p.off_tile_e + p.max_tiles;
    p.off_ntiles = p.off_tile_r0 + p.max_tiles;
}

}  // namespace

int64_t id_workspace_bytes(const IdProblem &p) { return 4 * (p.off_ntiles + 1); }

// Expected tiles per expert with BN-slot tiles when each token routes to
// n_used distinct experts of n_expert uniformly: an expert's slot count is
// binomial(n_tokens, n_used/n_expert), taken here as a normal distribution
// and summed over +-4 standard deviations.
double expected_tiles_per_expert(const IdProblem &p, int bn) {
    const double q = (double)p.n_used / (double)p.n_expert;
    const double mean = (double)p.n_tokens * (q < 1.0 ? q : 1.0);
    const double sd = std::sqrt(std::max(mean * (1.0 - (q < 1.0 ? q : 1.0)), 1e-9));
    const int lo = std::max(0, (int)std::floor(mean - 4 * sd)), hi = (int)std::ceil(mean + 4 * sd);
    double w_sum = 0, t_sum = 0;
    for (int c = lo; c <= hi; ++c) {
        const double z = (c - mean) / sd, w = std::exp(-0.5 * z * z);
        w_sum += w;
        t_sum += w * (double)((c + bn - 1) / bn);
    }
    return w_sum > 0 ? t_sum / w_sum : 1.0;
}

// Grouped-kernel configurations the automatic choice considers: 64 x 64,
// 128 x 80 and 128 x 128 tiles of 4 waves, and 128 x 128 and 128 x 96 tiles
// of 8 waves that each span all the slot rows (the others can be forced),
// with their rates in the grouped kernel (TileCfg::eff's unit).  The rates
// come from graph-timed launches of each configuration, forced, on 64 q4_K
// experts, 8 of 64 routed, 512 tokens (ne00 2560 x K 1024: 323 / 334 / 403 /
// 322 / 270 us; ne00 1024 x K 2560: 357 / 407 / 439 / 322 / 303 us, routing
// included), divided into the work the cost model below counts for each;
// partly filled tiles and the gathered slot columns make the wider slot
// tiles relatively slower here than in a dense OUT_PROD, except where every
// wave skips the same empty blocks.
struct IdAutoCfg {
    int cfg;
    double eff;
};
constexpr IdAutoCfg kIdAuto[] = {{4, 10.6}, {12, 8.35}, {0, 11.45}, {15, 14.5}, {17, 11.6}};

// l->variant on entry: forced configuration + 1 (an index into kCfgs that is
// built for the grouped kernel), or 0 for automatic.  The automatic choice
// minimizes the estimated time: workgroups x tile area x K / eff, slowed in
// proportion when there are fewer than 2560 waves (10 per CU: the CUs' MFMA
// pipes are not kept busy), with the workgroup count from the expected tiles
// per expert.  The shapes above run best with the 8-wave 128 x 96 tiles.
bool plan_id_back(IdProblem &p, Launch *l) {
    using namespace tiled;
    int best = -1;
    if (l->variant > 0) {
        for (int i = 0; i < kNumIdCfgs; ++i)
            if (kIdCfgs[i] == l->variant - 1) best = kIdCfgs[i];
        if (best < 0) return false;
    } else {
        double best_cost = 0;
        for (const IdAutoCfg &a : kIdAuto) {
            const TileCfg &c = kCfgs[a.cfg];
            const double wgs = (double)((p.M + c.bm() - 1) / c.bm()) * (double)p.n_expert *
                               expected_tiles_per_expert(p, c.bn());
            const double fill = std::min(1.0, wgs * (c.threads() / 64) / 2560.0);
            const double cost = wgs * c.bm() * c.bn() * (double)p.K / a.eff / fill;
            if (best < 0 || cost < best_cost) {
                best = a.cfg;
                best_cost = cost;
            }
        }
    }
    if (l->variant <= 0 && best == 17) {
        // 96-slot tiles: three 8-wave workgroups share a CU with 16-row
        // stages (78 VGPRs); with fewer than that per CU (about 16 waves)
        // the 32-row stages hide more of a stage's latency (64 q4_K experts,
        // 512 tokens: ne00 1024 x K 2560, 512 workgroups: 301 -> 286 us;
        // ne00 2560 x K 1024, 1280 workgroups: 268 -> 283 us the other way)
        const double wgs = (double)((p.M + 127) / 128) * (double)p.n_expert * expected_tiles_per_expert(p, 96);
        if (wgs * 8 < 24.0 * 256) best = 18;
    }
    const TileCfg &c = kCfgs[best];
    set_layout(p, c.bn());
    l->kernel = OUTPROD_KERNEL_TILED;
    l->variant = best;
    l->tile_m = c.bm();
    l->tile_n = c.bn();
    l->tile_k = c.bk;
    l->block = c.threads();
    l->lds_bytes = 2 * c.bk * (lds_ld(c.bm(), c.mf) + lds_ld(c.bn(), c.mf)) * 4 + 2 * c.bn() * 8;
    l->grid = ((p.M + c.bm() - 1) / c.bm()) * (int64_t)p.max_tiles;
    l->splits = 1;
    l->ksplit = p.K;
    return true;
}

hipError_t launch_id_back(const IdProblem &p, const Launch &l, hipStream_t s) {
    const void *fn = id_kernel_for(p.a_type, l.variant);
    if (!fn) return hipErrorInvalidValue;
    IdProblem pp = p;
    const int64_t slots = p.n_used * p.n_tokens;
    void *args1[] = {&pp};
    hipError_t e;
    if (slots <= kIdRouteFused) {
        e = hipLaunchKernel(id_route_for(slots), dim3(1), dim3(1024), args1, 0, s);
    } else {
        e = hipLaunchKernel((const void *)&id_rank_kernel, dim3((unsigned)p.rank_blocks), dim3(kIdRankBlock),
                            args1, 0, s);
        if (e == hipSuccess)
            e = hipLaunchKernel((const void *)&id_scan_kernel, dim3(1), dim3(1024), args1, 0, s);
        if (e == hipSuccess)
            e = hipLaunchKernel((const void *)&id_place_kernel, dim3((unsigned)((slots + 255) / 256)),
                                dim3(256), args1, 0, s);
    }
    if (e != hipSuccess) return e;
    int tiles_m = (int)((p.M + l.tile_m - 1) / l.tile_m);
    void *args[] = {&pp, &tiles_m};
    return hipLaunchKernel(fn, dim3((unsigned)l.grid), dim3(l.block), args, 0, s);
}

}  // namespace outprod
