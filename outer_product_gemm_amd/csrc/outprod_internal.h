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
};

// Launch configuration chosen by the planner.
struct Launch {
    int kernel;   // OUTPROD_KERNEL_*
    int variant;  // kernel-specific configuration index
    int tile_m, tile_n, tile_k;
    int block;
    int lds_bytes;
    int64_t grid;
};

// Per-kernel planning (host only, no HIP calls) and launching.
bool plan_skinny(const Problem &p, Launch *l);
bool plan_tiled(const Problem &p, Launch *l);
void plan_zero(const Problem &p, Launch *l);

hipError_t launch_skinny(const Problem &p, const Launch &l, hipStream_t s);
hipError_t launch_tiled(const Problem &p, const Launch &l, hipStream_t s);
hipError_t launch_zero(const Problem &p, const Launch &l, hipStream_t s);

}  // namespace outprod
