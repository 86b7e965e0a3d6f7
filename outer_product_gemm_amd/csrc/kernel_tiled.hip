// kernel_tiled.hip -- planning and launching of the tiled OUT_PROD kernel
// (the kernel and its configurations are in tiled_impl.h; each a type's
// instantiations are compiled in a tiled_*.hip file of their own).
#include <algorithm>

#include "tiled_impl.h"

namespace outprod {
namespace tiled {

// Rate unit of TileCfg::eff: tile area x K rows per microsecond on one CU,
// calibrated on the 27B q4_K shape (160 x 128 x 17408 per CU; 1647 us at eff
// 12.2 when calibrated, 1550 us since).  Only the ratios between
// configurations and against the split overheads below matter.
constexpr double kEffPerUs = 17.7e3;
// Split-K overheads: the reduce kernel's launch gap and its traffic (every
// partial read once, dst written once; the main kernel's extra partial writes
// are counted with them) at a sustained rate in bytes per microsecond.
constexpr double kSplitLaunchUs = 3.0;
constexpr double kSplitBytesPerUs = 4.0e6;

// A configuration's rate for a type.  The 80 x 256 tile (configuration 14)
// decodes half as much of a per flop as 160 x 128 and stages twice as much
// of b: measured faster for the K-quants with sub-block scales (m5120 k17408
// n1024: q3_K 1576 -> 1551 us, q4_K 1486 -> 1470, q5_K 1501 -> 1482, q6_K
// 1529 -> 1501), slower where the decode is cheap (f32 1359 -> 1437, f16
// 1384 -> 1429, bf16 1371 -> 1428) and about even for the other types.
//
// The 272 x 128 tile with loader waves (19: loads one stage ahead, 20: two)
// is faster than configuration 9 for every type at m17408 k5120 n1024; 20
// is the faster of the two for q4_0, q5_0 and q8_0 (1-2%), 19 for the
// others (20 runs one set for q3_K, q5_K and q6_K, whose second set spilled).
double cfg_eff(int cfg, int a_type) {
    const bool sub_scaled_k = a_type == OUTPROD_TYPE_Q3_K || a_type == OUTPROD_TYPE_Q4_K ||
                              a_type == OUTPROD_TYPE_Q5_K || a_type == OUTPROD_TYPE_Q6_K;
    const bool deep_loads = a_type == OUTPROD_TYPE_Q4_0 || a_type == OUTPROD_TYPE_Q5_0 ||
                            a_type == OUTPROD_TYPE_Q8_0;
    if (cfg == 14 && !sub_scaled_k) return 11.9;
    if (cfg == 19 && deep_loads) return 12.4;
    if (cfg == 20 && !deep_loads) return 12.4;
    return kCfgs[cfg].eff;
}

// Estimated time (us) of a configuration with `splits` K ranges: the
// busiest CU runs ceil(tiles * splits / 256) tiles of ksplit rows each --
// rounded up to whole stages, whose padding rows cost as much as real ones
// -- at the configuration's efficiency, plus the split's reduction.
double cfg_cost(int cfg, const Problem &p, int splits, int64_t ksplit) {
    const TileCfg &c = kCfgs[cfg];
    const int64_t tiles = ((p.M + c.bm() - 1) / c.bm()) * ((p.N + c.bn() - 1) / c.bn()) * p.ne12 * p.ne13;
    const int64_t per_cu = (tiles * splits + 255) / 256;
    const int64_t krows = ksplit < p.K ? ksplit : p.K;
    const int64_t kpad = (krows + c.bk - 1) / c.bk * c.bk;
    double t = (double)per_cu * c.bm() * c.bn() * (double)kpad / cfg_eff(cfg, p.a_type) / kEffPerUs;
    if (splits > 1)
        t += kSplitLaunchUs + (double)(2 * splits) * p.M * p.N * p.ne12 * p.ne13 * 4 / kSplitBytesPerUs;
    return t;
}

// Split counts the planner considers: each range at least 256 rows.
int max_splits(const Problem &p) {
    int64_t s = p.K / 256;
    if (s > 32) s = 32;
    while (s > 1 && split_bytes(p, (int)s) > kWorkspaceBytes) --s;
    return s < 1 ? 1 : (int)s;
}

}  // namespace tiled

using namespace tiled;

// l->variant on entry: forced configuration + 1, or 0 for automatic;
// l->splits on entry: forced split count, or 0 for automatic.
bool plan_tiled(const Problem &p, Launch *l) {
    int v = l->variant;
    int best, best_splits = 1;
    const int forced_splits = l->splits;
    if (forced_splits > 0) {
        if (forced_splits > 1 && split_bytes(p, forced_splits) > kWorkspaceBytes) return false;
        if (forced_splits > p.K) return false;
    }
    // candidate split counts: forced, or 1 .. max_splits
    const int s_lo = forced_splits > 0 ? forced_splits : 1;
    const int s_hi = forced_splits > 0 ? forced_splits : max_splits(p);
    const int c_lo = v > 0 ? v - 1 : 0, c_hi = v > 0 ? v - 1 : kNumAllCfgs - 1;
    if (v > 0 && !dense_cfg(v - 1)) return false;
    best = c_lo;
    double best_cost = 0;
    bool first = true;
    for (int i = c_lo; i <= c_hi; ++i) {
        if (!dense_cfg(i)) continue;  // the grouped kernel's tiles
        for (int sp = s_lo; sp <= s_hi; ++sp) {
            const int64_t ks = forced_splits > 0 ? (p.K + sp - 1) / sp : split_rows(p.K, sp);
            const double c = cfg_cost(i, p, sp, ks);
            if (first || c < best_cost) {
                best = i;
                best_splits = sp;
                best_cost = c;
                first = false;
            }
        }
    }
    const TileCfg &c = kCfgs[best];
    const int64_t tm = (p.M + c.bm() - 1) / c.bm(), tn = (p.N + c.bn() - 1) / c.bn();
    int64_t ksplit = p.K;
    if (best_splits > 1) {
        // forced counts split K evenly (any row count); automatic ones in
        // 64-row multiples, after which the count is what K needs
        ksplit = forced_splits > 0 ? (p.K + best_splits - 1) / best_splits : split_rows(p.K, best_splits);
        best_splits = (int)((p.K + ksplit - 1) / ksplit);
    }
    l->kernel = OUTPROD_KERNEL_TILED;
    l->variant = best;
    l->tile_m = c.bm();
    l->tile_n = c.bn();
    l->tile_k = c.bk;
    l->block = c.threads();
    l->lds_bytes = c.stages() * c.bk * (lds_ld(c.bm(), c.mf) + lds_ld(c.bn(), c.mf)) * 4;
    l->splits = best_splits;
    l->ksplit = best_splits > 1 ? ksplit : p.K;
    l->grid = tm * tn * p.ne12 * p.ne13 * best_splits;
    if (l->group_m <= 0) l->group_m = tile_group_m(p, *l, tm, tn);
    if (l->group_m > tm) l->group_m = (int)tm;
    return true;
}

// Tile order within a slice: consecutive logical tiles walk groups of
// group_m m-tiles (i0 fastest within a group, then i1, then the next group),
// so group_m = tiles_m walks i0 fastest over the slice and group_m = 1 walks
// i1 fastest.  Consecutive logical tiles run on one XCD (xcd_remap), whose
// L2 (4 MB) is shared by the tiles it runs at once -- about one per CU, 32 --
// and keeps little across rounds of tiles.  The estimate follows the
// kernel's mapping over each XCD's first (up to 4) rounds of 32 tiles: per round, the
// a strips (all of K, at a's stored size) of its distinct m-tiles plus the b
// strips of its distinct n-tiles.  Candidates: i0 fastest and groups of 1,
// 2, 4, ... m-tiles; the fewest bytes win (i0 fastest on ties).  Measured
// per launch with FETCH_SIZE: m5120 k17408 n1024 q4_K in 80 x 256 tiles (one
// round): 357 MB i0 fastest (estimate 342); m17408 k5120 in 272 x 128 tiles
// (two rounds): 523 MB i0 fastest, 400 MB i1 fastest (estimates 442 and 384
// MB); groups of 8 are estimated at 267 MB.
namespace {
int64_t tile_of(int64_t rem, int64_t g, int64_t tiles_m, int64_t tiles_n, int64_t *n) {
    const int64_t gsize = g * tiles_n, grp = rem / gsize, idx = rem % gsize;
    const int64_t gm = std::min(g, tiles_m - grp * g);
    *n = idx / gm;
    return grp * g + idx % gm;
}
}  // namespace

int tile_group_m(const Problem &p, const Launch &l, int64_t tiles_m, int64_t tiles_n) {
    const int64_t per = tiles_m * tiles_n;
    const int64_t chunk = ((int64_t)l.grid + 7) / 8;  // logical tiles per XCD
    const double a_strip = (p.nb01 > 0 ? (double)p.nb01 / (double)p.M : 4.0) * l.tile_m;
    const double b_strip = 4.0 * l.tile_n;
    int64_t best = tiles_m;
    double best_bytes = 0;
    bool first = true;
    int64_t cand[64];
    int nc = 0;
    cand[nc++] = tiles_m;
    for (int64_t g = 1; g < tiles_m && nc < 64; g *= 2) cand[nc++] = g;
    for (int ci = 0; ci < nc; ++ci) {
        const int64_t g = cand[ci];
        double bytes = 0;
        for (int64_t x = 0; x < 8; ++x) {
            const int64_t lo = x * chunk, hi = std::min<int64_t>((x + 1) * chunk, l.grid);
            for (int64_t r0 = lo; r0 < hi && r0 < lo + 4 * 32; r0 += 32) {
                int64_t ms[32], ns[32];
                int cnt = 0;
                for (int64_t t = r0; t < std::min(r0 + 32, hi); ++t, ++cnt) {
                    // strips of different slices (and K ranges) are different data
                    const int64_t zz = t / per;
                    ms[cnt] = zz * tiles_m + tile_of(t % per, g, tiles_m, tiles_n, &ns[cnt]);
                    ns[cnt] += zz * tiles_n;
                }
                std::sort(ms, ms + cnt);
                std::sort(ns, ns + cnt);
                const int64_t dm = std::unique(ms, ms + cnt) - ms, dn = std::unique(ns, ns + cnt) - ns;
                bytes += (double)dm * a_strip + (double)dn * b_strip;
            }
        }
        if (first || bytes < best_bytes * (1.0 - 1e-9)) {
            best = g;
            best_bytes = bytes;
        }
        first = false;
    }
    return (int)std::min<int64_t>(best, 127);
}

hipError_t launch_tiled(const Problem &p, const Launch &l, hipStream_t s) {
    int tiles_m = (int)((p.M + l.tile_m - 1) / l.tile_m);
    int tiles_n = (int)((p.N + l.tile_n - 1) / l.tile_n);
    int group_m = l.group_m;
    Problem pp = p;
    void *args[] = {&pp, &tiles_m, &tiles_n, &group_m};
    const void *fn = nullptr;
    switch (p.a_type) {
    case OUTPROD_TYPE_F32: fn = tiled_kernel_f32(p.a_type, l.variant, p.b_kt); break;
    case OUTPROD_TYPE_F16:
    case OUTPROD_TYPE_BF16: fn = tiled_kernel_half(p.a_type, l.variant, p.b_kt); break;
    case OUTPROD_TYPE_Q8_0:
    case OUTPROD_TYPE_Q4_0:
    case OUTPROD_TYPE_Q4_1: fn = tiled_kernel_q8(p.a_type, l.variant, p.b_kt); break;
    case OUTPROD_TYPE_Q5_0:
    case OUTPROD_TYPE_Q5_1: fn = tiled_kernel_q45(p.a_type, l.variant, p.b_kt); break;
    case OUTPROD_TYPE_Q4_K:
    case OUTPROD_TYPE_Q2_K: fn = tiled_kernel_k4(p.a_type, l.variant, p.b_kt); break;
    case OUTPROD_TYPE_Q3_K:
    case OUTPROD_TYPE_Q5_K:
    case OUTPROD_TYPE_Q6_K: fn = tiled_kernel_k(p.a_type, l.variant, p.b_kt); break;
    default: break;
    }
    if (!fn) return hipErrorInvalidValue;
    return hipLaunchKernel(fn, dim3((unsigned)l.grid), dim3(l.block), args, 0, s);
}

}  // namespace outprod
