// outprod_internal.h -- what the host side hands to the kernel launchers.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace outprod {

// One validated OUT_PROD problem.  Strides are in bytes.  a is addressed
// row by row: row (k, i02, i03) starts at a + k*nb01 + i02*nb02 + i03*nb03.
struct Problem {
    const uint8_t *a;
    const uint8_t *b;
    uint8_t *dst;
    int a_type;
    int64_t M;            // ne00 (a's width, dst dim 0)
    int64_t N;            // ne10 (b's width, dst dim 1)
    int64_t K;            // contraction length
    int64_t nb01, nb02, nb03;
    int64_t nb10, nb11, nb12, nb13;  // b: nb10 == 4 (row-major) or nb11 == 4 (b_kt)
    int64_t nb0, nb1, nb2, nb3;      // dst: nb0 == 4 except in an operand-swapped problem
    int64_t ne12, ne13;              // dst slices
    int64_t dps2, dps3;              // broadcast ratios
    bool vec_a;    // f32 a: base and strides 16-byte aligned
    bool vec_b;    // b: base and strides (other than the contiguous one) 16-byte aligned
    bool b_kt;     // b's K dim is the contiguous one (a transposed view)
    bool bcast_b;  // the dps2/dps3 slice broadcast applies to the kernel's b
                   // operand (operand-swapped problem), not to a
    // Split K: splits > 1 runs the contraction as `splits` ranges of ksplit
    // rows (the last one shorter); range s writes its partial dst, dense
    // [slices][N][M] fp32, at ws + s * M*N*slices*4, and the reduce kernel
    // adds the partials in range order into dst.
    int splits;
    int64_t ksplit;
    uint8_t *ws;
};

// Bytes of one workspace of the library's pool; split plans never need more.
constexpr int64_t kWorkspaceBytes = 64ll << 20;
// Workspaces per device at most (each bound to one stream at a time).
constexpr int kMaxWorkspaces = 4;
// Bytes of the allocation-free entry point's static device scratch.
constexpr int64_t kScratchBytes = 32ll << 20;

// Workspace bytes a split plan needs (0 without a split).
inline int64_t split_bytes(const Problem &p, int splits) {
    return splits > 1 ? (int64_t)splits * p.M * p.N * p.ne12 * p.ne13 * 4 : 0;
}

// Launch configuration chosen by the planner.
struct Launch {
    int kernel;   // OUTPROD_KERNEL_*
    int variant;  // kernel-specific configuration index
    int tile_m, tile_n, tile_k;
    int block;
    int lds_bytes;
    int64_t grid;     // main kernel workgroups (all splits)
    int splits;       // 1 = no split
    int64_t ksplit;   // rows per split
    int group_m;      // tiled kernel: tiles walk groups of group_m m-tiles within
                      // a slice (i0 fastest inside a group); on entry to
                      // plan_tiled, 0 = automatic
};

// A validated OUT_PROD call and its plan.  swapped: the problem runs with
// the operands exchanged (a narrow f32 b with a wide f32 a).
struct Checked {
    Problem p;
    Launch l;
    bool swapped;
};

// Every host-side check of the contract, then the plan (no HIP call).
// kernel: out_prod_ex's override code (0 = automatic); no_split: plan
// without a K split unless one is forced.  Returns OUTPROD_OK or a status.
int validate_and_plan(const void *a, int a_type, const float *b, const float *dst,
                      const int64_t *ne, const int64_t *nb, int kernel, Checked *c,
                      bool no_split = false);
// Enqueue a validated plan on stream s; ws: the split's partials
// (split_bytes(c.p, c.l.splits) bytes), unused without a split.
hipError_t enqueue(Checked &c, hipStream_t s, uint8_t *ws);

// One validated MUL_MAT_ID_BACK problem: for routed slot s = i + n_used*t,
// dst row (i, t) = expert ids[i,t] (ne00 x K, rows of ne00 values along K)
// times the slot's gradient column g[:, i, t] (K contiguous floats).
struct IdProblem {
    const uint8_t *as;    // experts: row r of expert e at as + e*nb02 + r*nb01
    const uint8_t *g;     // g(r, i, t) at g + 4r + i*nbg1 + t*nbg2
    const uint8_t *ids;   // int32 ids[i, t] at ids + 4i + t*nbi1
    uint8_t *dst;         // dst(c, i, t) at dst + 4c + i*nbd1 + t*nbd2
    int a_type;
    int64_t M, K;         // ne00, expert rows
    int64_t n_expert, n_used, n_tokens;
    int64_t nb01, nb02, nbg1, nbg2, nbi1, nbd1, nbd2;
    bool vec_a, vec_g;
    // routing tables in the workspace (int32 offsets from ws)
    uint8_t *ws;
    int bn;               // slots per tile of the grouped kernel
    int rank_blocks;      // blocks of the rank kernel (1024 slots each)
    int max_tiles;        // tile-table capacity: ceil(slots / bn) + n_expert
    int64_t off_rank, off_hist, off_offsets, off_sorted, off_tile_e, off_tile_r0, off_ntiles;
};

// Limits of MUL_MAT_ID_BACK: experts per op (the rank kernel's LDS tables).
constexpr int kIdMaxExperts = 512;
constexpr int kIdRankBlock = 1024;  // slots per rank-kernel block (16 waves)
constexpr int kIdRouteFused = 16384;  // most slots routed by the one-block kernel

bool plan_id_back(IdProblem &p, Launch *l);   // sets the tile config and table layout
int64_t id_workspace_bytes(const IdProblem &p);
hipError_t launch_id_back(const IdProblem &p, const Launch &l, hipStream_t s);

// Per-kernel planning (host only, no HIP calls) and launching.
bool plan_skinny(const Problem &p, Launch *l);
bool plan_tiled(const Problem &p, Launch *l);
int tile_group_m(const Problem &p, const Launch &l, int64_t tiles_m, int64_t tiles_n);
void plan_zero(const Problem &p, Launch *l);

hipError_t launch_skinny(const Problem &p, const Launch &l, hipStream_t s);
hipError_t launch_tiled(const Problem &p, const Launch &l, hipStream_t s);
hipError_t launch_zero(const Problem &p, const Launch &l, hipStream_t s);
hipError_t launch_split_reduce(const Problem &p, hipStream_t s);

// K rows per split for `splits` ranges: a multiple of 64 (keeps 16-byte
// alignment of K-contiguous b and whole MFMA stages).
inline int64_t split_rows(int64_t K, int splits) {
    const int64_t r = (K + splits - 1) / splits;
    return (r + 63) / 64 * 64;
}

}  // namespace outprod
