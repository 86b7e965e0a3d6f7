// kernel_reduce.hip -- second pass of a split-K OUT_PROD: dst = the sum of
// the per-range partial results, added in range order (range 0 first), so a
// split launch is as deterministic as an unsplit one.  Partials are dense
// [splits][slices][N][M] fp32 in the workspace; dst is written through its
// own strides (nb0 may differ from 4 in an operand-swapped problem).
#include "kernel_common.h"

namespace outprod {
namespace {

// One thread per 4 consecutive i0 of one (slice, i1) row.  vec_ws: M % 4 ==
// 0, so a thread's partials are 16-byte aligned; vec_dst: dst rows and
// strides 16-byte aligned with nb0 == 4.
__global__ __launch_bounds__(256) void split_reduce_kernel(Problem p, int groups_per_row, int rows,
                                                           int vec_ws, int vec_dst) {
    const int M = (int)p.M, N = (int)p.N, ne12 = (int)p.ne12;
    const int64_t split_floats = (int64_t)rows * M;  // one range's partial block
    const float *ws = (const float *)p.ws;
    const int total = rows * groups_per_row;
    for (int g = blockIdx.x * blockDim.x + threadIdx.x; g < total; g += gridDim.x * blockDim.x) {
        const int row = g / groups_per_row;
        const int i0 = 4 * (g % groups_per_row);
        const int z = row / N, i1 = row % N;
        const float *src = ws + (int64_t)row * M + i0;
        floatx4 acc;
        if (vec_ws) {
            // the partials of up to 8 ranges are loaded together (clamped
            // indices, no branch), then added in range order
            acc = *(const floatx4 *)src;
            for (int sp = 1; sp < p.splits; sp += 8) {
                floatx4 v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int r = sp + u < p.splits ? sp + u : p.splits - 1;
                    v[u] = *(const floatx4 *)(src + r * split_floats);
                }
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (sp + u < p.splits) acc += v[u];
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float v = 0.f;
                if (i0 + e < M) {
                    v = src[e];
                    for (int sp = 1; sp < p.splits; ++sp) v += src[e + sp * split_floats];
                }
                acc[e] = v;
            }
        }
        uint8_t *d = p.dst + (int64_t)(z % ne12) * p.nb2 + (int64_t)(z / ne12) * p.nb3 +
                     (int64_t)i1 * p.nb1 + (int64_t)i0 * p.nb0;
        if (vec_dst && i0 + 3 < M) {
            *(floatx4 *)d = acc;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (i0 + e < M) *(float *)(d + (int64_t)e * p.nb0) = acc[e];
        }
    }
}

}  // namespace

hipError_t launch_split_reduce(const Problem &p, hipStream_t s) {
    const int64_t groups_per_row = (p.M + 3) / 4;
    const int64_t rows = p.N * p.ne12 * p.ne13;
    const int64_t total = groups_per_row * rows;
    int gpr = (int)groups_per_row, nrows = (int)rows;
    int vec_ws = p.M % 4 == 0;
    int vec_dst = p.nb0 == 4 && (uintptr_t)p.dst % 16 == 0 && p.nb1 % 16 == 0 && p.nb2 % 16 == 0 &&
                  p.nb3 % 16 == 0;
    int64_t grid = (total + 255) / 256;
    if (grid > 8192) grid = 8192;
    Problem pp = p;
    void *args[] = {&pp, &gpr, &nrows, &vec_ws, &vec_dst};
    return hipLaunchKernel((const void *)&split_reduce_kernel, dim3((unsigned)grid), dim3(256), args, 0,
                           s);
}

}  // namespace outprod
