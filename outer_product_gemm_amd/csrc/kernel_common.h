// kernel_common.h -- device-side helpers shared by the OUT_PROD kernels.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "outprod_internal.h"

namespace outprod {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// Workgroup -> logical tile remap so that consecutive logical tiles run on the
// same XCD.  The MI355X's 8 XCDs each have their own L2 and the dispatcher
// deals workgroups to them round-robin; neighbouring tiles share cache lines
// (skinny kernel) or operand panels (tiled kernel).  Bijective for any grid.
__device__ __forceinline__ int xcd_remap(int bid, int grid) {
    const int nx = 8;
    const int xcd = bid % nx, local = bid / nx;
    const int per = grid / nx, rem = grid % nx;
    return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

// IEEE binary16 bits (the low 16 of h) -> float.  Every binary16 value,
// subnormals included, is exactly a binary32 value, and the hardware
// conversion (v_cvt_f32_f16) is exact: half denormals are kept in the default
// float mode.  Inf/NaN keep their class.
__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Grouped-head broadcast: dst slice z = i2 + ne12*i3 reads a slice
// (i2/dps2, i3/dps3) and b slice (i2, i3).
struct SliceBase {
    const uint8_t *a;
    const uint8_t *b;
    uint8_t *dst;
};

__device__ __forceinline__ SliceBase slice_base(const Problem &p, int z) {
    // 32-bit index math (the host guarantees slice counts below 2^31); 64-bit
    // division would expand into long instruction sequences.
    const int ne12 = (int)p.ne12, dps2 = (int)p.dps2, dps3 = (int)p.dps3;
    const int i2 = z % ne12, i3 = z / ne12;
    const int i02 = i2 / dps2, i03 = i3 / dps3;
    SliceBase s;
    if (p.bcast_b) {  // operand-swapped problem: the broadcast side is b
        s.a = p.a + (int64_t)i2 * p.nb02 + (int64_t)i3 * p.nb03;
        s.b = p.b + (int64_t)i02 * p.nb12 + (int64_t)i03 * p.nb13;
    } else {
        s.a = p.a + (int64_t)i02 * p.nb02 + (int64_t)i03 * p.nb03;
        s.b = p.b + (int64_t)i2 * p.nb12 + (int64_t)i3 * p.nb13;
    }
    s.dst = p.dst + (int64_t)i2 * p.nb2 + (int64_t)i3 * p.nb3;
    return s;
}

// Split K: narrow problem q (a copy of the launch's problem) and slice s to
// contraction range `sp` -- rows [sp*ksplit, min(K, (sp+1)*ksplit)) -- whose
// partial result goes to the dense [slices][N][M] block sp of the workspace.
__device__ __forceinline__ void apply_split(Problem &q, SliceBase &s, int z, int sp) {
    const int64_t kb = (int64_t)sp * q.ksplit;
    const int64_t klen = q.K - kb < q.ksplit ? q.K - kb : q.ksplit;
    s.a += kb * q.nb01;
    s.b += kb * q.nb11;
    const int64_t plane = q.M * q.N;
    s.dst = q.ws + ((int64_t)sp * q.ne12 * q.ne13 + z) * plane * 4;
    q.K = klen;
    // K-contiguous b moves by kb floats: vector loads along k stay aligned
    // only for kb a multiple of 4 (row-major b and a move by whole rows)
    if (q.b_kt && (kb & 3) != 0) q.vec_b = false;
    q.nb0 = 4;
    q.nb1 = 4 * q.M;
}

__device__ __forceinline__ float ldf(const uint8_t *p) { return *(const float *)p; }

// x, hidden from the optimizer's known-bits analysis (an empty asm with x as
// its in/out operand; no instruction is emitted).  For a dword of masked
// codes it keeps byte e's conversion a single v_cvt_f32_ubyte{e} instead of a
// bit-field extract of the known-nonzero bits plus a conversion.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
    asm("" : "+v"(x));
    return x;
}

}  // namespace outprod
